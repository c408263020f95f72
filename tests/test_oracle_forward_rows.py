"""Pins of the oracle's row-wise entry point, forward_rows (no GPU needed).

forward_rows is the checker behind every fused GPU test, so it is tied here
to things other than itself:

* forward(), the whole-tensor composition of the separately pinned steps,
  row by row: decode (one query per sequence), chunked queries (Lq < Lk),
  prefill (Lq = Lk), FP8 index inputs with distinct per-row scales, and
  caches allocated longer than the context;
* a hand-worked end-to-end fixture (tests/golden/tiny_forward.json) through
  scores, top-k and attention for two queries of a four-token context, and a
  hand-worked FP8 decode row;
* mutants: copies of forward_rows with one plausible mistake each (a wrong
  visible count, another query's or sequence's scale bytes, the cache length
  taken for the context, another sequence's latent rows) must each fail at
  least one of the pins above.
"""
import inspect
import json
import math
import os

import numpy as np
import pytest

from oracle import dsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "tiny_forward.json")) as f:
        return json.load(f)


def _tiny_scores():
    with open(os.path.join(GOLDEN, "tiny_scores.json")) as f:
        return json.load(f)


_LN = {"ln2": math.log(2.0), "ln3": math.log(3.0), "ln4": math.log(4.0), "ln4/3": math.log(4.0 / 3.0)}


def _num(x):
    return _LN[x] if isinstance(x, str) else float(x)


def _arr(x):
    return np.vectorize(_num, otypes=[np.float64])(np.array(x, dtype=object))


# ------------------------------------------------------------------ cases ----
def _rand_inputs(seed, B, Lq, Lk, H=3, D=8, NH=2, Dqk=6, Dv=4, fp8=False, cache_extra=0):
    """Random inputs; caches hold Lk + cache_extra rows (the tail is garbage)."""
    r = np.random.default_rng(seed)
    Lc = Lk + cache_extra
    if fp8:
        # codes drawn from the finite E4M3 values (0x7F / 0xFF are NaN), distinct scale bytes per row
        q = r.integers(0, 0x7F, (B, Lq, H, D)) | (r.integers(0, 2, (B, Lq, H, D)) << 7)
        k = r.integers(0, 0x7F, (B, Lc, D)) | (r.integers(0, 2, (B, Lc, D)) << 7)
        q, k = q.astype(np.uint8), k.astype(np.uint8)
        qs = r.integers(118, 136, (B, Lq, H)).astype(np.uint8)
        ks = r.integers(118, 136, (B, Lc)).astype(np.uint8)
    else:
        q, k = r.standard_normal((B, Lq, H, D)), r.standard_normal((B, Lc, D))
        qs = ks = None
    w = r.standard_normal((B, Lq, H))
    qa = r.standard_normal((B, Lq, NH, Dqk))
    kv = r.standard_normal((B, Lc, Dqk))
    return dict(q_idx=q, q_scale=qs, k_idx=k, k_scale=ks, head_w=w, q_attn=qa, kv=kv, Lq=Lq, Lk=Lk, Dv=Dv)


CASES = {
    "decode": dict(seed=1, B=3, Lq=1, Lk=29),
    "chunked": dict(seed=2, B=2, Lq=5, Lk=23),
    "prefill": dict(seed=3, B=2, Lq=12, Lk=12),
    "fp8_chunked": dict(seed=4, B=2, Lq=4, Lk=19, fp8=True),
    "fp8_decode": dict(seed=5, B=3, Lq=1, Lk=17, fp8=True),
}
K_SEL = 4
SCALE = 0.37


def _pin_equals_forward(fr, case, kv_len_arg=True):
    """forward_rows(fr) equals forward() row by row; caches may be longer than Lk."""
    c = _rand_inputs(**case)
    Lq, Lk = c["Lq"], c["Lk"]
    # forward() sees caches trimmed to the context
    trim = lambda a: None if a is None else a[:, :Lk]  # noqa: E731
    ref = O.forward(c["q_idx"], c["q_scale"], trim(c["k_idx"]), trim(c["k_scale"]), c["head_w"], c["q_attn"],
                    trim(c["kv"]), K_SEL, SCALE, c["Dv"])
    B = c["q_idx"].shape[0]
    rows = [(b, i) for b in range(B) for i in range(Lq)]
    kw = dict(kv_len=Lk) if kv_len_arg else {}
    got = fr(c["q_idx"], c["q_scale"], c["k_idx"], c["k_scale"], c["head_w"], c["q_attn"], c["kv"], rows, Lq,
             K_SEL, SCALE, c["Dv"], **kw)
    for (b, i), g in zip(rows, got):
        n = O.visible_count(Lq, Lk, i)
        if g["scores"].shape != (n,):
            return False
        if not np.array_equal(g["scores"], ref["scores"][b, i, :n]):
            return False
        if not np.array_equal(g["topk"], ref["topk"][b, i]):
            return False
        if not (np.array_equal(g["out"], ref["out"][b, i]) and np.array_equal(g["lse"], ref["lse"][b, i])):
            return False
    return True


def _pin_golden_bf16(fr):
    """Hand-worked two-query forward through scores, top-k and attention."""
    s, g = _tiny_scores(), _golden()["bf16_path"]
    q = np.array(s["q_idx"], dtype=np.float64)[None]
    w = np.array(s["head_w"], dtype=np.float64)[None]
    k = np.array(s["k_idx"], dtype=np.float64)[None]
    qa = _arr(g["q_attn"])[None]
    kv = _arr(g["kv"])[None]
    rows = [(0, 0), (0, 1)]
    got = fr(q, None, k, None, w, qa, kv, rows, s["q_len"], g["topk_k"], g["scale"], g["v_dim"])
    for i, r in enumerate(got):
        n = O.visible_count(s["q_len"], s["kv_len"], i)
        exp_sc = [v for v in s["scores"][i][:n]]
        if r["scores"].shape != (n,) or not np.array_equal(r["scores"], np.array(exp_sc, dtype=np.float64)):
            return False
        if [int(j) for j in r["topk"]] != g["topk"][i]:
            return False
        if np.abs(r["out"] - np.array(g["out"][i], dtype=np.float64)).max() > 1e-12:
            return False
        if np.abs(r["lse"] - _arr(g["lse"][i])).max() > 1e-12:
            return False
    return True


def _pin_golden_fp8(fr):
    """Hand-worked FP8 decode row: codes and ue8m0 scale bytes decoded by row."""
    g = _golden()["fp8_path"]
    q = np.array(g["q_codes"], dtype=np.uint8)[None]          # [1, 1, H, D]
    qs = np.array(g["q_scale"], dtype=np.uint8)[None]         # [1, 1, H]
    k = np.array(g["k_codes"], dtype=np.uint8)[None]          # [1, 3, D]
    ks = np.array(g["k_scale"], dtype=np.uint8)[None]         # [1, 3]
    w = np.array(g["head_w"], dtype=np.float64)[None]
    qa = np.zeros((1, 1, 1, 2))
    kv = np.arange(6, dtype=np.float64).reshape(1, 3, 2)
    r = fr(q, qs, k, ks, w, qa, kv, [(0, 0)], 1, g["topk_k"], 1.0, 1)[0]
    return np.array_equal(r["scores"], np.array(g["scores"])) and [int(j) for j in r["topk"]] == g["topk"]


def _try(f):
    try:
        return f()
    except (IndexError, ValueError):
        return False                           # a shape error is also a caught mistake


def _all_pins(fr):
    res = {name: _try(lambda case=case: _pin_equals_forward(fr, case)) for name, case in CASES.items()}
    res["long_caches"] = _try(lambda: _pin_equals_forward(fr, dict(seed=6, B=2, Lq=3, Lk=21, cache_extra=9)))
    res["long_caches_fp8"] = _try(lambda: _pin_equals_forward(fr, dict(seed=7, B=2, Lq=1, Lk=15, fp8=True,
                                                                        cache_extra=6)))
    res["golden_bf16"] = _try(lambda: _pin_golden_bf16(fr))
    res["golden_fp8"] = _try(lambda: _pin_golden_fp8(fr))
    return res


# ------------------------------------------------------------------ tests ----
@pytest.mark.parametrize("name", list(CASES))
def test_forward_rows_equals_forward(name):
    assert _pin_equals_forward(O.forward_rows, CASES[name])


def test_forward_rows_with_caches_longer_than_context():
    assert _pin_equals_forward(O.forward_rows, dict(seed=6, B=2, Lq=3, Lk=21, cache_extra=9))
    assert _pin_equals_forward(O.forward_rows, dict(seed=7, B=2, Lq=1, Lk=15, fp8=True, cache_extra=6))


def test_forward_rows_default_context_is_cache_length():
    assert _pin_equals_forward(O.forward_rows, CASES["chunked"], kv_len_arg=False)


def test_forward_rows_hand_worked_two_queries():
    assert _pin_golden_bf16(O.forward_rows)


def test_forward_rows_hand_worked_fp8_row():
    assert _pin_golden_fp8(O.forward_rows)


def test_golden_forward_fixture_through_forward():
    """The same fixture through the whole-tensor forward()."""
    s, g = _tiny_scores(), _golden()["bf16_path"]
    res = O.forward(np.array(s["q_idx"], dtype=np.float64)[None], None, np.array(s["k_idx"], dtype=np.float64)[None],
                    None, np.array(s["head_w"], dtype=np.float64)[None], _arr(g["q_attn"])[None], _arr(g["kv"])[None],
                    g["topk_k"], g["scale"], g["v_dim"])
    assert res["topk"][0].tolist() == g["topk"]
    np.testing.assert_allclose(res["out"][0], np.array(g["out"], dtype=np.float64), rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["lse"][0], _arr(g["lse"]), rtol=0, atol=1e-12)


# One plausible mistake per mutant, planted in a copy of forward_rows (CPU only).
MUTANTS = {
    "visible_count_ignores_context": ("n = visible_count(q_len, Lk, i)", "n = visible_count(q_len, q_len, i)"),
    "query_scales_of_query_0": ("dequant_rows(q_idx[b, i], q_scale[b, i])", "dequant_rows(q_idx[b, i], q_scale[b, 0])"),
    "key_scales_of_sequence_0": ("dequant_rows(k_idx[b], k_scale[b])", "dequant_rows(k_idx[b], k_scale[0])"),
    "context_from_cache_length": ("Lk = kb.shape[0] if kv_len is None else kv_len", "Lk = kb.shape[0]"),
    "latent_rows_of_sequence_0": ("np.asarray(kv[b], dtype=np.float64)", "np.asarray(kv[0], dtype=np.float64)"),
    "query_heads_reversed": ("qi = np.asarray(q_idx[b, i], dtype=np.float64)",
                             "qi = np.asarray(q_idx[b, i][::-1], dtype=np.float64)"),
}


def _mutant(old, new):
    src = inspect.getsource(O.forward_rows)
    assert src.count(old) == 1, old
    ns = dict(vars(O))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)  # noqa: S102  (test-only code mutation)
    return ns["forward_rows"]


def test_pins_pass_on_the_oracle():
    res = _all_pins(O.forward_rows)
    assert all(res.values()), res


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_mutant(name):
    res = _all_pins(_mutant(*MUTANTS[name]))
    assert not all(res.values()), f"mutant {name} passed every pin"
