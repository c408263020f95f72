"""GPU: the filtered decode top-k inside dsa_forward (the indexer lists each
2048-key chunk's highest-scoring keys; the top-k selects from the lists, or
from the full row when the lists cannot hold the selection) against the
one-work-group-per-row selection of dsa_topk over the same scores, bit for
bit.  The oracle's selection on those scores is the same set by the
standalone top-k's own parity tests; here the check is that filtering
changes nothing, including on inputs built so that the lists fail."""
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


def _forward_vs_full_row(cfg, inp, expect_slots=None):
    dsa = _dsa()
    p = dsa.make_problem(cfg)
    slots = dsa.topk_list_slots(p)
    assert slots > 0, "shape does not take the filtered top-k"
    if expect_slots is not None:
        assert slots == expect_slots
    scores = dsa.index_scores(p, inp["q_idx"], inp["q_scale"], inp["k_idx"], inp["k_scale"], inp["head_w"])
    full = dsa.topk(p, scores)
    idx = torch.empty(cfg.batch, cfg.q_len, cfg.topk, dtype=torch.int32, device=DEV)
    dsa.forward(p, inp["q_idx"], inp["q_scale"], inp["k_idx"], inp["k_scale"], inp["head_w"], inp["q_attn"],
                inp["kv"], topk_idx=idx)
    torch.cuda.synchronize()
    assert torch.equal(idx, full), cfg.name
    return idx, scores


@pytest.mark.parametrize("B,Lq,Lk,K,slots", [
    (32, 1, 32768, 2048, 256),       # the 32K decode shape: 16 chunks
    (3, 1, 30721, 2048, 256),        # 16 chunks, the last holding one key
    (2, 1, 40000, 2048, 256),        # ragged last chunk
    (2, 4, 33000, 2048, 256),        # four causal queries per sequence: the earlier rows end
                                     # inside the last chunk, chunks past a row's end list nothing
    (8, 1, 131072, 2048, 128),       # the 128K decode shape: 64 chunks of 128 slots
    (1, 1, 262144, 2048, 64),        # 128 chunks
    (2, 1, 65536, 4096, 256),        # the largest K the lists serve
    (2, 1, 65536, 1, 256),           # K = 1
    (3, 2, 50001, 777, 256),
])
def test_forward_list_topk_equals_full_row(B, Lq, Lk, K, slots):
    cfg = C.scaled(C.DECODE_32K, name=f"lists_B{B}_q{Lq}_L{Lk}_K{K}", batch=B, q_len=Lq, kv_len=Lk, topk=K,
                   plant_count=min(300, Lk // 100))
    _forward_vs_full_row(cfg, generate(cfg, device=DEV), slots)


def test_forward_list_topk_fp8_index():
    # FP8 index keys (ue8m0 row scales) at 32K: the FP8 decode kernel's lists
    cfg = C.scaled(C.PREFILL_64K_FP8, name="lists_fp8_B4_L32768", batch=4, q_len=1, kv_len=32768)
    _forward_vs_full_row(cfg, generate(cfg, device=DEV), 256)


def _planted_direction(inp, b, i, D):
    """sum_h w_h q_h of query (b, i), rescaled to norm 3 sqrt(D): keys along it score high."""
    q = inp["q_idx"][b, i].float()
    u = (inp["head_w"][b, i].float()[:, None] * q).sum(0)
    return u * (3.0 * D ** 0.5 / u.norm())


@pytest.mark.parametrize("kind", ["one_chunk", "four_chunks", "all_equal", "tail_chunk"])
def test_forward_list_topk_fallback(kind):
    """Inputs whose top K crowd into fewer chunks than the lists can carry
    (or that hold one repeated key): the lists cannot hold the selection,
    the top-k falls back to the full row, and the result stays exact."""
    B, Lk, K, D = 2, 32768, 2048, 128
    cfg = C.scaled(C.DECODE_32K, name=f"lists_fallback_{kind}", batch=B, q_len=1, kv_len=Lk, topk=K,
                   plant_count=0)
    inp = generate(cfg, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(1234)
    for b in range(B):
        u = _planted_direction(inp, b, 0, D)
        if kind == "all_equal":
            inp["k_idx"][b] = inp["k_idx"][b, 7].clone()            # one key everywhere: every score ties
            continue
        if kind == "one_chunk":
            spans = [(2048 * 5, 2048 * 6)]                          # all of chunk 5 scores high
        elif kind == "four_chunks":
            spans = [(2048 * c, 2048 * (c + 1)) for c in (1, 6, 9, 14)]
        else:
            spans = [(Lk - 2048, Lk)]                               # the most recent chunk
        for s0, s1 in spans:
            z = torch.randn(s1 - s0, D, generator=g, device=DEV)
            inp["k_idx"][b, s0:s1] = (u[None, :] + 0.5 * z).to(inp["k_idx"].dtype)
    idx, _ = _forward_vs_full_row(cfg, inp, 256)
    if kind == "one_chunk":
        # nearly every chosen position lies in the planted chunk (far more than its list holds)
        assert float(((idx >= 2048 * 5) & (idx < 2048 * 6)).float().mean()) > 0.95
    if kind == "all_equal":
        # ties go to the lower positions
        assert torch.equal(idx[:, 0], torch.arange(K, dtype=torch.int32, device=DEV).expand(B, K))
