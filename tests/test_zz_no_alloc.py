"""GPU: dsa_forward_static, the forward that works in the library's static
per-GPU scratch array instead of a caller workspace, against dsa_forward
with a caller workspace on the same inputs.

Both run the same plan and the same kernels, so outputs, LSEs and top-k
indices must agree bit for bit.  Calls come in pairs, the second with a
smaller input, so the second runs on scratch the first left full of its own
state (histograms, barrier counters, partials of a larger problem)."""
import pytest
import torch

from dsa_workloads import configs as C
from dsa_workloads import generate

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import sparse_attention_15_amd as dsa
    dsa.lib()
    yield


def _dsa():
    import sparse_attention_15_amd as dsa
    return dsa


def _both(cfg, with_idx):
    """(workspace forward, static forward) results for cfg, in that order."""
    dsa = _dsa()
    p = dsa.make_problem(cfg)
    inp = generate(cfg, device=DEV)
    args = (inp["q_idx"], inp["q_scale"], inp["k_idx"], inp["k_scale"], inp["head_w"], inp["q_attn"], inp["kv"])
    res = []
    for static in (False, True):
        odt = torch.float32 if cfg.attn_dtype == "f32" else torch.bfloat16
        out = torch.empty(cfg.batch, cfg.q_len, cfg.attn_heads, cfg.v_dim, dtype=odt, device=DEV)
        lse = torch.empty(cfg.batch, cfg.q_len, cfg.attn_heads, dtype=torch.float32, device=DEV)
        idx = (torch.empty(cfg.batch, cfg.q_len, cfg.topk, dtype=torch.int32, device=DEV) if with_idx else None)
        torch.cuda.synchronize()
        if static:
            before = torch.cuda.memory_allocated()
            dsa.forward_static(p, *args, out=out, lse=lse, topk_idx=idx)
            assert torch.cuda.memory_allocated() == before      # nothing allocated for the call
        else:
            dsa.forward(p, *args, out=out, lse=lse, topk_idx=idx)
        torch.cuda.synchronize()
        res.append((out, lse, idx))
    return p, res


def _same(cfg, with_idx=True):
    dsa = _dsa()
    p, ((o0, l0, i0), (o1, l1, i1)) = _both(cfg, with_idx)
    assert torch.equal(o0.view(torch.uint8), o1.view(torch.uint8)), cfg.name
    assert torch.equal(l0, l1), cfg.name
    if with_idx:
        assert torch.equal(i0, i1), cfg.name
    return dsa.topk_list_slots(p), dsa.topk_slice_len(p)


# top-k plans: candidate lists (16 or more 2048-key chunks), sliced (few
# long rows with K beyond the lists), one work-group per row (short rows)
SMALL_LISTS = C.scaled(C.DECODE_32K, name="decode_bf16_B2_ctx40000", batch=2, kv_len=40000)
SMALL_SLICED = C.scaled(C.DECODE_128K, name="decode_bf16_B2_ctx70001_K8192", batch=2, kv_len=70001, topk=8192)
SMALL_DECODE = C.scaled(C.DECODE_32K, name="decode_bf16_B4_ctx9000", batch=4, kv_len=9000)


def test_static_forward_decode_32k_then_smaller():
    # 32 x 32K (candidate lists), then 2 x 70001 with K = 8192 (sliced
    # top-k) and 2 x 40000 (lists again, over the sliced selection's state)
    assert _same(C.DECODE_32K) == (256, 0)
    lists, sl = _same(SMALL_SLICED)
    assert lists == 0 and sl > 0
    assert _same(SMALL_LISTS) == (256, 0)


def test_static_forward_decode_128k_then_smaller():
    # 8 x 128K (candidate lists of 128 slots left in the scratch), then
    # 2 x 70001 sliced, 2 x 40000 with lists and 4 x 9000 without indices out
    assert _same(C.DECODE_128K) == (128, 0)
    assert _same(SMALL_SLICED)[1] > 0
    assert _same(SMALL_LISTS)[0] == 256
    assert _same(SMALL_DECODE, with_idx=False) == (0, 0)


SMALL_PREFILL = C.scaled(C.PREFILL_8K, name="prefill_bf16_L300_ctx700", batch=2, q_len=300, kv_len=700)


def test_static_forward_small_prefills():
    # fp32 and bf16 prefill shapes after the decode pairs above
    _same(C.TINY)
    _same(SMALL_PREFILL)
