"""The fused forward captured in a HIP graph and replayed.

A decode step is launch-bound at small batch, so a caller may capture the
whole path (index scores, top-k, sparse attention, split combine) once and
replay it per step with fresh inputs copied into the captured buffers.  The
library makes no allocation, memset or synchronisation inside the forward, so
the captured launches are the eager ones; these tests check that every replay,
with eager work and synchronisations between replays, gives exactly the eager
result for the inputs then in the buffers, for decode shapes (split lists
and the combine launch) and prefill shapes.
"""
import pytest
import torch

from dsa_workloads import configs as C
from dsa_workloads import generate

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

NAMES = ("q_idx", "q_scale", "k_idx", "k_scale", "head_w", "q_attn", "kv")

CASES = {
    # 3 splits per query at 5000 keys, bf16 index path.
    "decode_b3_L5000": C.scaled(C.DECODE_32K, name="decode_b3_L5000", batch=3, kv_len=5000, plant_count=50),
    # FP8 index path, several splits.
    "decode128k_b2_L9000": C.scaled(C.DECODE_128K, name="decode128k_b2_L9000", batch=2, kv_len=9000,
                                    plant_count=16),
    # prefill-shaped launches: rows shorter and longer than K, no split
    "prefill_q77_L3000": C.scaled(C.PREFILL_8K, name="prefill_q77_L3000", q_len=77, kv_len=3000),
    "fp8_prefill_q40_L3000": C.scaled(C.PREFILL_64K_FP8, name="fp8_prefill_q40_L3000", q_len=40, kv_len=3000),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import sparse_attention_15_amd as dsa
    dsa.lib()
    yield


def _same(a, b):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


@pytest.mark.parametrize("name", list(CASES))
def test_forward_graph_replay_matches_eager(name):
    import sparse_attention_15_amd as dsa
    cfg = CASES[name]
    p = dsa.make_problem(cfg)
    first = generate(cfg, device=DEV, set_index=0)
    static = {k: (first[k].clone() if first[k] is not None else None) for k in NAMES}
    out_dt = torch.float32 if p.out_dtype == dsa.DSA_F32 else torch.bfloat16
    out = torch.empty(cfg.batch, cfg.q_len, cfg.attn_heads, cfg.v_dim, dtype=out_dt, device=DEV)
    lse = torch.empty(cfg.batch, cfg.q_len, cfg.attn_heads, dtype=torch.float32, device=DEV)
    idx = torch.empty(cfg.batch, cfg.q_len, cfg.topk, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(dsa.workspace_size(p, dsa.DSA_OP_FORWARD), 1), dtype=torch.uint8, device=DEV)

    def step():
        dsa.forward(p, *(static[k] for k in NAMES), out=out, lse=lse, topk_idx=idx, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for set_index in (1, 2, 0, 3):
        fresh = generate(cfg, device=DEV, set_index=set_index)
        for k in NAMES:
            if static[k] is not None:
                static[k].copy_(fresh[k])
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        idx.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        g_out, g_lse, g_idx = out.clone(), lse.clone(), idx.clone()

        # Eager call on buffers of its own, between replays.
        e_lse = torch.empty_like(lse)
        e_idx = torch.empty_like(idx)
        e_out, e_lse, e_idx = dsa.forward(p, *(fresh[k] for k in NAMES), lse=e_lse, topk_idx=e_idx)
        torch.cuda.synchronize()
        assert _same(g_idx, e_idx), f"{name} set {set_index}: top-k differs from eager"
        assert _same(g_out, e_out), f"{name} set {set_index}: output differs from eager"
        assert _same(g_lse, e_lse), f"{name} set {set_index}: lse differs from eager"
        assert bool(torch.isfinite(g_out.float()).all())
        assert int(g_idx.min()) >= -1


def test_forwards_on_two_streams_equal_sequential_calls():
    # the library keeps no mutable global state: two calls in flight on two
    # streams (default priority) give what each gives alone
    import sparse_attention_15_amd as dsa
    cfg_a = CASES["decode_b3_L5000"]
    cfg_b = CASES["prefill_q77_L3000"]
    res = {}
    for cfg in (cfg_a, cfg_b):
        inp = generate(cfg, device=DEV, set_index=5)
        p = dsa.make_problem(cfg)
        lse = torch.empty(cfg.batch, cfg.q_len, cfg.attn_heads, dtype=torch.float32, device=DEV)
        idx = torch.empty(cfg.batch, cfg.q_len, cfg.topk, dtype=torch.int32, device=DEV)
        ws = torch.empty(max(dsa.workspace_size(p, dsa.DSA_OP_FORWARD), 1), dtype=torch.uint8, device=DEV)
        out, lse, idx = dsa.forward(p, *(inp[k] for k in NAMES), lse=lse, topk_idx=idx, workspace=ws)
        torch.cuda.synchronize()
        res[cfg.name] = (inp, p, ws, out.clone(), lse.clone(), idx.clone())
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = {}
    torch.cuda.synchronize()
    for _ in range(3):
        for st, cfg in zip(streams, (cfg_a, cfg_b)):
            inp, p, ws, *_ = res[cfg.name]
            with torch.cuda.stream(st):
                lse = torch.empty(cfg.batch, cfg.q_len, cfg.attn_heads, dtype=torch.float32, device=DEV)
                idx = torch.empty(cfg.batch, cfg.q_len, cfg.topk, dtype=torch.int32, device=DEV)
                got[cfg.name] = dsa.forward(p, *(inp[k] for k in NAMES), lse=lse, topk_idx=idx, workspace=ws)
        torch.cuda.synchronize()
        for cfg in (cfg_a, cfg_b):
            _, _, _, out, lse, idx = res[cfg.name]
            g_out, g_lse, g_idx = got[cfg.name]
            assert _same(g_idx, idx) and _same(g_out, out) and _same(g_lse, lse), cfg.name
