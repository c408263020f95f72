"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each test ties the oracle to a hand-worked fixture, a closed form, an
invariant the pages state or imply, a brute force, or a library routine, so
that a dropped term, a wrong sign or index or a transposed operand in the
oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import dsa_oracle as O
from dsa_workloads import configs as C
from dsa_workloads import generate, random_score_rows, quantize_e4m3_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _num(x):
    return {"-0": -0.0, "+0": 0.0}.get(x, x) if isinstance(x, str) else x


# ---------------------------------------------------------------- scores ----
def test_golden_scores_and_topk():
    g = _load("tiny_scores.json")
    q = np.array(g["q_idx"], dtype=np.float64)[None]
    w = np.array(g["head_w"], dtype=np.float64)[None]
    k = np.array(g["k_idx"], dtype=np.float64)[None]
    sc = O.index_scores(q, k, w, g["q_len"], g["kv_len"])[0]
    exp = np.array([[np.nan if v is None else v for v in row] for row in g["scores"]])
    for i in range(g["q_len"]):
        n = O.visible_count(g["q_len"], g["kv_len"], i)
        np.testing.assert_array_equal(sc[i, :n], exp[i, :n])
        assert np.all(np.isneginf(sc[i, n:]))
    for kk, sets in g["topk"].items():
        idx = O.topk(sc[None], g["q_len"], g["kv_len"], int(kk))[0]
        for i in range(g["q_len"]):
            got = [int(j) for j in idx[i] if j >= 0]
            assert got == sets[i], (kk, i, got)
            assert all(j == -1 for j in idx[i][len(got):])


def _rand_case(seed, B=2, Lq=5, Lk=9, H=3, D=4):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, Lq, H, D)), r.standard_normal((B, Lk, D)),
            r.standard_normal((B, Lq, H)), Lq, Lk)


def test_scores_head_permutation_invariant():
    q, k, w, Lq, Lk = _rand_case(1)
    perm = np.array([2, 0, 1])
    a = O.index_scores(q, k, w, Lq, Lk)
    b = O.index_scores(q[:, :, perm], k, w[:, :, perm], Lq, Lk)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


def test_scores_positive_weight_scaling():
    q, k, w, Lq, Lk = _rand_case(2)
    a = O.index_scores(q, k, w, Lq, Lk)
    b = O.index_scores(q, k, 3.5 * w, Lq, Lk)
    fin = np.isfinite(a)
    np.testing.assert_allclose(b[fin], 3.5 * a[fin], rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(O.topk(a, Lq, Lk, 3), O.topk(b, Lq, Lk, 3))


def test_scores_relu_is_per_head_not_after_sum():
    # one key, two heads with opposite dot products: the gate kills the
    # negative head before weighting, so the score is w0 * x0, not w0*x0 + w1*x1
    q = np.array([[[[1.0, 0.0], [-1.0, 0.0]]]])
    k = np.array([[[2.0, 0.0]]])
    w = np.array([[[1.0, 1.0]]])
    assert O.index_scores(q, k, w, 1, 1)[0, 0, 0] == 2.0
    w2 = np.array([[[1.0, -1.0]]])   # negative weight on the silenced head changes nothing
    assert O.index_scores(q, k, w2, 1, 1)[0, 0, 0] == 2.0
    w3 = np.array([[[-1.0, 1.0]]])   # negative weight on the live head flips the sign
    assert O.index_scores(q, k, w3, 1, 1)[0, 0, 0] == -2.0


def _hadamard(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h / math.sqrt(n)


def test_scores_hadamard_rotation_invariant():
    # HF model doc, DSA item 1: the rotation applied before FP8 is orthogonal,
    # so rotating both q and k leaves every dot product, hence every score, unchanged.
    q, k, w, Lq, Lk = _rand_case(3, D=8)
    Hm = _hadamard(8)
    np.testing.assert_allclose(Hm @ Hm.T, np.eye(8), atol=1e-15)
    a = O.index_scores(q, k, w, Lq, Lk)
    b = O.index_scores(q @ Hm.T, k @ Hm.T, w, Lq, Lk)
    fin = np.isfinite(a)
    np.testing.assert_allclose(b[fin], a[fin], rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.isfinite(b), fin)


def test_scores_causality():
    # appending future tokens (keys and queries) leaves earlier rows unchanged
    q, k, w, Lq, Lk = _rand_case(4, Lq=6, Lk=6)
    full = O.index_scores(q, k, w, Lq, Lk)
    part = O.index_scores(q[:, :4], k[:, :4], w[:, :4], 4, 4)
    np.testing.assert_array_equal(full[:, :4, :4], part)
    assert np.all(np.isneginf(full[:, 3, 4:]))
    # the diagonal is visible: query i sees key i
    assert np.all(np.isfinite(np.diagonal(full, axis1=1, axis2=2)))


def test_scores_decode_sees_whole_cache():
    q, k, w, _, Lk = _rand_case(5, Lq=1, Lk=7)
    sc = O.index_scores(q, k, w, 1, Lk)
    assert np.all(np.isfinite(sc))


def test_scores_against_explicit_loops():
    # brute force with scalar loops on a tiny case (independent of the matmul form)
    q, k, w, Lq, Lk = _rand_case(6, B=1, Lq=3, Lk=4, H=2, D=3)
    sc = O.index_scores(q, k, w, Lq, Lk)
    for i in range(Lq):
        for s in range(Lk):
            if s > Lk - Lq + i:
                continue
            tot = 0.0
            for h in range(2):
                dot = sum(q[0, i, h, d] * k[0, s, d] for d in range(3))
                tot += w[0, i, h] * (dot if dot > 0 else 0.0)
            assert abs(sc[0, i, s] - tot) < 1e-13


# ----------------------------------------------------------------- top-k ----
def test_golden_select_16_top4():
    g = _load("select_16_top4.json")
    for name, qd in g["queries"].items():
        row = np.array([_num(x) for x in qd["scores"]], dtype=np.float64)
        got = O.topk_row(row, len(row), g["k"])
        assert list(got) == qd["expected"], name


def _topk_bruteforce(row, n, k):
    items = sorted(range(n), key=lambda s: (-float(row[s]), s))
    chosen = sorted(items[:min(k, n)])
    return chosen + [-1] * (k - len(chosen))


@pytest.mark.parametrize("tie_fraction,neg_zero", [(0.0, False), (0.3, False), (0.2, True)])
def test_topk_against_bruteforce(tie_fraction, neg_zero):
    rows = random_score_rows(12, 300, seed=77, tie_fraction=tie_fraction, neg_zero=neg_zero).numpy()
    for r in range(rows.shape[0]):
        n = 300 - 17 * r
        for k in (1, 7, 64, 299, 400):
            assert list(O.topk_row(rows[r], n, k)) == _topk_bruteforce(rows[r], n, k)


def test_topk_short_rows_take_everything():
    row = np.array([5.0, -1.0, 2.0])
    assert list(O.topk_row(row, 3, 8)) == [0, 1, 2, -1, -1, -1, -1, -1]
    assert list(O.topk_row(row, 2, 2)) == [0, 1]


# ------------------------------------------------------------- attention ----
def test_golden_attention():
    g = _load("tiny_attention.json")
    ln = {"ln3": math.log(3.0), "ln4": math.log(4.0)}
    rows = np.array([[ln.get(x, x) for x in r] for r in g["kv_rows"]], dtype=np.float64)
    q = np.array(g["q_attn"], dtype=np.float64)
    for case in g["cases"]:
        out, lse = O.sparse_attention_row(q, rows, np.array(case["selected"]), case["scale"], g["v_dim"])
        if "out" in case:
            assert abs(out[0, 0] - case["out"]) < 1e-13
            assert abs(lse[0] - ln[case["lse"]]) < 1e-13
        else:
            e25, r3 = math.exp(25.0), math.sqrt(3.0)
            assert abs(out[0, 0] - (10 + 2 * r3 + 1000 * e25) / (1 + r3 + e25)) < 1e-9
            assert abs(lse[0] - math.log(1 + r3 + e25)) < 1e-12


def _attn_case(seed, B=2, Lq=6, Lk=10, NH=3, Dqk=7, Dv=5):
    r = np.random.default_rng(seed)
    return r.standard_normal((B, Lq, NH, Dqk)), r.standard_normal((B, Lk, Dqk)), Lq, Lk, Dv


def test_attention_k_ge_n_equals_dense_causal():
    qa, kv, Lq, Lk, Dv = _attn_case(10)
    scale = 1 / math.sqrt(7)
    # select everything visible: K >= n for every row
    idx = np.stack([np.stack([O.topk_row(np.zeros(Lk), O.visible_count(Lq, Lk, i), Lk)
                              for i in range(Lq)]) for _ in range(2)])
    out, lse = O.sparse_attention(qa, kv, idx, scale, Dv)
    out_d, lse_d = O.dense_masked_attention(qa, kv, idx, Lq, Lk, scale, Dv)
    np.testing.assert_allclose(out, out_d, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_d, rtol=1e-12, atol=1e-13)
    # library routine: torch's fp64 scaled_dot_product_attention with a boolean causal mask
    q_t = torch.from_numpy(qa).permute(0, 2, 1, 3)                        # B, NH, Lq, Dqk
    k_t = torch.from_numpy(kv)[:, None].expand(-1, 3, -1, -1)             # MQA: shared rows
    v_t = torch.from_numpy(kv[..., :Dv])[:, None].expand(-1, 3, -1, -1)
    allowed = torch.ones(Lq, Lk, dtype=torch.bool).tril(Lk - Lq)
    ref = torch.nn.functional.scaled_dot_product_attention(q_t, k_t, v_t, attn_mask=allowed, scale=scale)
    np.testing.assert_allclose(out, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-11, atol=1e-12)


def test_attention_sparse_equals_dense_masked_for_partial_sets():
    qa, kv, Lq, Lk, Dv = _attn_case(11)
    r = np.random.default_rng(12)
    sc = r.standard_normal((2, Lq, Lk))
    idx = O.topk(sc, Lq, Lk, 3)
    out, lse = O.sparse_attention(qa, kv, idx, 0.3, Dv)
    out_d, lse_d = O.dense_masked_attention(qa, kv, idx, Lq, Lk, 0.3, Dv)
    np.testing.assert_allclose(out, out_d, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_d, rtol=1e-12, atol=1e-13)


def test_attention_single_key_returns_its_value_row():
    qa, kv, _, _, Dv = _attn_case(13, B=1, Lq=1)
    out, lse = O.sparse_attention_row(qa[0, 0], kv[0], np.array([4, -1]), 0.7, Dv)
    np.testing.assert_array_equal(out, np.broadcast_to(kv[0, 4, :Dv], out.shape))
    np.testing.assert_allclose(lse, 0.7 * qa[0, 0] @ kv[0, 4], rtol=1e-14)


def test_attention_equal_logits_give_mean_of_rows():
    _, kv, _, _, Dv = _attn_case(14, B=1)
    sel = np.array([1, 3, 8, -1])
    out, lse = O.sparse_attention_row(np.zeros((3, 7)), kv[0], sel, 1.0, Dv)
    np.testing.assert_allclose(out[0], kv[0, [1, 3, 8], :Dv].mean(axis=0), rtol=1e-14)
    np.testing.assert_allclose(lse, math.log(3.0), rtol=1e-15)


def test_attention_values_are_leading_dims_and_convex():
    qa, kv, _, _, Dv = _attn_case(15, B=1)
    sel = np.array([0, 2, 5, 9])
    out, _ = O.sparse_attention_row(qa[0, 0], kv[0], sel, 0.5, Dv)
    lo = kv[0, sel, :Dv].min(axis=0)
    hi = kv[0, sel, :Dv].max(axis=0)
    assert np.all(out >= lo - 1e-12) and np.all(out <= hi + 1e-12)


def test_lse_against_scipy_logsumexp():
    qa, kv, _, _, Dv = _attn_case(16, B=1)
    sel = np.array([0, 1, 2, 6, 9])
    _, lse = O.sparse_attention_row(qa[0, 0], kv[0], sel, 0.4, Dv)
    z = 0.4 * qa[0, 0] @ kv[0, sel].T
    np.testing.assert_allclose(lse, scipy.special.logsumexp(z, axis=1), rtol=1e-14)


# ------------------------------------------------------------------ fp8 -----
def test_e4m3_decode_matches_torch_float8_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan) and nan.sum() == 2
    np.testing.assert_array_equal(mine[~nan], ref[~nan])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9


def test_ue8m0_and_generator_quantiser():
    x = torch.randn(64, 128, generator=torch.Generator().manual_seed(5), dtype=torch.float32)
    x[3] = 0.0
    codes, exps = quantize_e4m3_rows(x)
    deq = O.dequant_rows(codes.numpy(), exps.numpy())
    scale = O.ue8m0_decode(exps.numpy())
    amax = x.abs().amax(1).double().numpy()
    nz = amax > 0
    # the scale is the smallest power of two with amax/scale <= 448
    assert np.all(amax[nz] / scale[nz] <= 448.0) and np.all(amax[nz] / (scale[nz] / 2) > 448.0)
    assert exps[3] == 127 and np.all(deq[3] == 0)
    # RNE on a 3-bit mantissa: relative error at most 2^-4 for normals
    err = np.abs(deq - x.double().numpy())
    assert np.all(err <= np.abs(x.double().numpy()) * 2.0 ** -4 + scale[:, None] * 2.0 ** -10)


# ------------------------------------------------------------- workload -----
def test_tiny_workload_planted_keys_are_selected():
    cfg = C.TINY
    inp = generate(cfg)
    res = O.forward(inp["q_idx"].numpy(), None, inp["k_idx"].numpy(), None, inp["head_w"].numpy(),
                    inp["q_attn"].numpy(), inp["kv"].numpy(), cfg.topk, cfg.softmax_scale, cfg.v_dim)
    # later queries overwrite earlier plantings: only the last writer of a key keeps its plant
    last = {}
    for i, pos in enumerate(inp["planted"][0]):
        for s in pos:
            last[s] = i
    hit = tot = 0
    for s, i in last.items():
        chosen = set(int(j) for j in res["topk"][0, i] if j >= 0)
        tot += 1
        hit += s in chosen
    assert tot >= 150 and hit / tot > 0.9, (hit, tot)


def test_band_check_rule():
    r = np.random.default_rng(20)
    row = r.standard_normal(100)
    ref = O.topk_row(row, 100, 10)
    ok, swaps, _ = O.topk_band_check(row, ref, 100, 10)
    assert ok and swaps == 0
    # swap the 10th-best for the 11th-best: accepted only if their gap is inside the band
    order = np.argsort(-row, kind="stable")
    bad = np.sort(np.concatenate([order[:9], order[10:11]]))
    gap = row[order[9]] - row[order[10]]
    ok, _, _ = O.topk_band_check(row, bad, 100, 10, rel_eps=1e-6)
    assert ok == (gap <= 1e-6 * np.abs(row).max())
    ok, swaps, _ = O.topk_band_check(row, bad, 100, 10, rel_eps=2 * gap / np.abs(row).max())
    assert ok and swaps == 1
    ok, _, _ = O.topk_band_check(row, ref[:9], 100, 10)
    assert not ok
