"""Cache append and a multi-step decode loop on the GPU, through the C ABI.

Caches are allocated with room for more tokens than the current context
(kv_capacity > kv_len); each decode step appends one token per sequence and
runs the fused path for one query at the grown context.  Step t of a loop
that starts at context L0 is row t of the causal problem with Lq = T queries
and Lk = L0 + T keys, which is what the oracle computes."""
import numpy as np
import pytest
import torch

from dsa_workloads import configs as C
from dsa_workloads import generate
from oracle import dsa_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    yield


def _dsa():
    import sparse_attention_15_amd as dsa
    return dsa


def np64(t):
    if t is None:
        return None
    return t.cpu().numpy() if t.dtype == torch.uint8 else t.float().cpu().numpy().astype(np.float64)


CASES = {
    "f32_tiny": C.scaled(C.TINY, name="loop_f32", q_len=4, kv_len=130, plant_count=2),
    "bf16_decode": C.scaled(C.DECODE_32K, name="loop_bf16", batch=2, q_len=4, kv_len=3004, plant_count=30),
    "fp8_decode": C.scaled(C.PREFILL_64K_FP8, name="loop_fp8", batch=2, q_len=4, kv_len=2600),
}


def _caches(cfg, full, cap, filled):
    """Caches of `cap` tokens per sequence holding the first `filled` tokens of `full`."""
    def mk(t, tail):
        c = torch.zeros((cfg.batch, cap) + tail, dtype=t.dtype, device=DEV)
        c[:, :filled] = t[:, :filled]
        return c
    k = mk(full["k_idx"], (cfg.index_dim,))
    ks = mk(full["k_scale"], ()) if full["k_scale"] is not None else None
    kv = mk(full["kv"], (cfg.qk_dim,))
    return k, ks, kv


@pytest.mark.parametrize("name", list(CASES))
def test_append_writes_exactly_the_new_rows(name):
    dsa = _dsa()
    cfg = CASES[name]
    full = generate(cfg, device=DEV)
    T = cfg.q_len
    L0 = cfg.kv_len - T
    cap = cfg.kv_len + 7
    k, ks, kv = _caches(cfg, full, cap, L0)
    p = dsa.make_problem(C.scaled(cfg, q_len=1, kv_len=L0), kv_capacity=cap)
    sl = slice(L0, L0 + T)
    dsa.cache_append(p, full["k_idx"][:, sl].contiguous(),
                     full["k_scale"][:, sl].contiguous() if ks is not None else None,
                     full["kv"][:, sl].contiguous(), k, ks, kv)
    torch.cuda.synchronize()
    assert torch.equal(k[:, :cfg.kv_len].view(torch.uint8), full["k_idx"].view(torch.uint8))
    assert torch.equal(kv[:, :cfg.kv_len].view(torch.uint8), full["kv"].view(torch.uint8))
    assert torch.count_nonzero(kv[:, cfg.kv_len:].view(torch.uint8)) == 0       # nothing beyond
    if ks is not None:
        assert torch.equal(ks[:, :cfg.kv_len], full["k_scale"])


@pytest.mark.parametrize("name", list(CASES))
def test_forward_with_spare_capacity_matches_compact_caches(name):
    dsa = _dsa()
    cfg = CASES[name]
    full = generate(cfg, device=DEV)
    cap = cfg.kv_len + 33
    k, ks, kv = _caches(cfg, full, cap, cfg.kv_len)

    def run(p, kk, kks, kkv):
        lse = torch.empty(cfg.batch, cfg.q_len, cfg.attn_heads, dtype=torch.float32, device=DEV)
        idx = torch.empty(cfg.batch, cfg.q_len, cfg.topk, dtype=torch.int32, device=DEV)
        out, lse, idx = dsa.forward(p, full["q_idx"], full["q_scale"], kk, kks, full["head_w"], full["q_attn"], kkv,
                                    lse=lse, topk_idx=idx)
        torch.cuda.synchronize()
        return out, lse, idx

    a = run(dsa.make_problem(cfg), full["k_idx"], full["k_scale"], full["kv"])
    b = run(dsa.make_problem(cfg, kv_capacity=cap), k, ks, kv)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.int32 else x,
                           y.view(torch.uint8) if y.dtype != torch.int32 else y)


@pytest.mark.parametrize("name", list(CASES))
def test_decode_loop_matches_causal_rows(name):
    dsa = _dsa()
    cfg = CASES[name]
    full = generate(cfg, device=DEV)
    T = cfg.q_len
    L0 = cfg.kv_len - T
    cap = cfg.kv_len
    k, ks, kv = _caches(cfg, full, cap, L0)
    host = {kk: np64(v) for kk, v in full.items() if kk != "planted"}
    ref = O.forward_rows(host["q_idx"], host["q_scale"], host["k_idx"], host["k_scale"], host["head_w"],
                         host["q_attn"], host["kv"], [(b, t) for b in range(cfg.batch) for t in range(T)],
                         cfg.q_len, cfg.topk, cfg.softmax_scale, cfg.v_dim)
    ref = {(r_b, r_t): r for (r_b, r_t), r in zip([(b, t) for b in range(cfg.batch) for t in range(T)], ref)}
    tol = 1e-4 if cfg.attn_dtype == "f32" else 2e-2
    for t in range(T):
        step = C.scaled(cfg, q_len=1, kv_len=L0 + t)
        dsa.cache_append(dsa.make_problem(step, kv_capacity=cap), full["k_idx"][:, L0 + t:L0 + t + 1].contiguous(),
                         full["k_scale"][:, L0 + t:L0 + t + 1].contiguous() if ks is not None else None,
                         full["kv"][:, L0 + t:L0 + t + 1].contiguous(), k, ks, kv)
        p = dsa.make_problem(C.scaled(cfg, q_len=1, kv_len=L0 + t + 1), kv_capacity=cap)
        q = lambda x: None if x is None else x[:, t:t + 1].contiguous()  # noqa: E731
        lse = torch.empty(cfg.batch, 1, cfg.attn_heads, dtype=torch.float32, device=DEV)
        idx = torch.empty(cfg.batch, 1, cfg.topk, dtype=torch.int32, device=DEV)
        out, lse, idx = dsa.forward(p, q(full["q_idx"]), q(full["q_scale"]), k, ks, q(full["head_w"]),
                                    q(full["q_attn"]), kv, lse=lse, topk_idx=idx)
        torch.cuda.synchronize()
        for b in range(cfg.batch):
            r = ref[(b, t)]
            n = L0 + t + 1
            sel = idx[b, 0].cpu().numpy()
            ok, swaps, msg = O.topk_band_check(r["scores"], sel, n, cfg.topk)
            assert ok, f"step {t} seq {b}: {msg}"
            ref_o, ref_l = r["out"], r["lse"]
            if swaps:
                # the oracle's attention step on the GPU's own set (it differs inside the band)
                ref_o, ref_l = O.sparse_attention_row(host["q_attn"][b, t], host["kv"][b], sel, cfg.softmax_scale,
                                                      cfg.v_dim)
            assert np.abs(np64(out[b, 0]) - ref_o).max() <= tol, f"step {t} seq {b}"
            assert np.abs(lse[b, 0].cpu().numpy() - ref_l).max() <= tol, f"step {t} seq {b}"
