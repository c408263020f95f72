"""GPU: the sliced top-k (few long rows, one work-group per row slice, three
launches) against the oracle's selection, bit for bit, and against the
one-work-group-per-row kernel inside the fused forward."""
import numpy as np
import pytest
import torch

from dsa_workloads import configs as C
from dsa_workloads import generate, random_score_rows
from oracle import dsa_oracle as O

from test_gpu_parity import _special_rows

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


def _check(scores, B, Lq, Lk, K):
    dsa = _dsa()
    cfg = C.scaled(C.DECODE_32K, batch=B, q_len=Lq, kv_len=Lk, topk=K)
    p = dsa.make_problem(cfg)
    assert dsa.workspace_size(p, dsa.DSA_OP_TOPK) > 0, "shape does not take the sliced path"
    idx = dsa.topk(p, scores, workspace="auto")
    single = dsa.topk(p, scores)
    torch.cuda.synchronize()
    assert torch.equal(idx, single)
    got, host = idx.cpu().numpy(), scores.cpu().numpy()
    for b in range(B):
        for i in range(Lq):
            ref = O.topk_row(host[b, i], O.visible_count(Lq, Lk, i), K)
            assert np.array_equal(got[b, i], ref), (b, i)


@pytest.mark.parametrize("shape", [
    # (B, Lq, Lk, K, stride_pad, ties, negzero)
    (8, 1, 131072, 2048, 0, 0.1, True),      # the 128K decode shape: 32 slices of 4096, one launch
    (3, 1, 70001, 2048, 0, 0.2, True),       # slices of 1024, ragged last slice, rows on different XCDs
    (2, 3, 66000, 64, 3, 0.3, True),         # unaligned row stride: scalar loads; causal rows
    (1, 2, 100000, 2048, 0, 0.0, False),
    (5, 1, 65536, 65535, 0, 0.5, True),      # K = n - 1
    (4, 1, 80000, 1, 0, 0.9, True),          # K = 1 with massive ties
    (2, 4, 65537, 65535, 0, 0.0, False),     # rows of 65534..65537 positions around K
    (128, 1, 131072, 2048, 0, 0.1, False),   # 4096 work-groups: more than the GPU holds at once,
                                             # so the three-launch form runs instead of one launch
])
def test_sliced_topk_bitexact(shape):
    B, Lq, Lk, K, pad, ties, nz = shape
    stride = Lk + pad
    rows = random_score_rows(B * Lq, stride, seed=Lk * 3 + K, device=DEV, tie_fraction=ties, neg_zero=nz)
    _check(rows.view(B, Lq, stride).contiguous(), B, Lq, Lk, K)


@pytest.mark.parametrize("kind", ["inf", "outliers", "narrow", "equal", "two_values", "subnormal", "huge_range",
                                  "pivot_ties"])
@pytest.mark.parametrize("Lk,K", [(70000, 2048), (100000, 100), (80000, 2048), (65536, 5000)])
def test_sliced_topk_special_rows(kind, Lk, K):
    B, Lq = 1, 2
    scores = _special_rows(kind, B * Lq, Lk, seed=Lk + K + 1).view(B, Lq, Lk).contiguous()
    _check(scores, B, Lq, Lk, K)


@pytest.mark.parametrize("B,Lq,Lk", [(8, 1, 131072), (2, 1, 70001), (2, 3, 66000), (1, 1, 100000), (16, 1, 65536)])
def test_forward_sliced_topk_equals_single_workgroup(B, Lq, Lk):
    """dsa_forward's indices (sliced selection on its own scores: K = 6000
    is beyond the indexer's candidate lists) equal the one-work-group-per-row
    selection of dsa_topk over the same scores."""
    dsa = _dsa()
    cfg = C.scaled(C.DECODE_32K, batch=B, q_len=Lq, kv_len=Lk, topk=6000, plant_count=min(300, Lk // 100))
    inp = generate(cfg, device=DEV)
    p = dsa.make_problem(cfg)
    assert dsa.topk_slice_len(p) > 0 and dsa.topk_list_slots(p) == 0
    scores = dsa.index_scores(p, inp["q_idx"], inp["q_scale"], inp["k_idx"], inp["k_scale"], inp["head_w"])
    single = dsa.topk(p, scores)
    idx = torch.empty(B, Lq, cfg.topk, dtype=torch.int32, device=DEV)
    dsa.forward(p, inp["q_idx"], inp["q_scale"], inp["k_idx"], inp["k_scale"], inp["head_w"], inp["q_attn"],
                inp["kv"], topk_idx=idx)
    torch.cuda.synchronize()
    assert torch.equal(idx, single)
