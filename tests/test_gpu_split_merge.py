"""GPU: decode-shaped attention splits each query's list over work-groups,
which store partial outputs (in the output's precision) and LSEs that a
second kernel merges in fp32.  The merged result must agree with the
unsplit computation of the same rows to the rounding of the bf16
probabilities; a bf16 output, whose partials are rounded to bf16 before the
merge, must stay within that double rounding of the fp32 output; reruns
must be bit-identical."""
import numpy as np
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


def _case(big_batch, lk, k, seed):
    """big_batch sequences; the first two are the rows compared."""
    cfg = C.scaled(C.DECODE_32K, name="split_merge", batch=big_batch, kv_len=lk, topk=k, plant_count=0)
    inp = generate(cfg, device=DEV)
    g = torch.Generator().manual_seed(seed)
    idx = torch.stack([torch.sort(torch.randperm(lk, generator=g)[:k]).values for _ in range(big_batch)])
    return cfg, inp, idx.view(big_batch, 1, k).to(torch.int32).to(DEV)


# two rows split 16 (2048 keys), 4 (512) or 2 (300) ways
@pytest.mark.parametrize("lk,k", [(4096, 2048), (9000, 2048), (3000, 512), (3000, 300)])
def test_split_merge_against_unsplit(lk, k):
    """Split and unsplit launches round the bf16 probabilities of the PV
    product against different running maxima, so they agree to that
    rounding: each output is within 2^-9 (half a bf16 step) of
    sum_j p_j v_j / sum_j p_j in relative terms per probability, so the two
    differ by at most 2^-8 * max |v| over the chosen rows; the LSEs (fp32
    sums of unrounded probabilities) agree to fp32 rounding."""
    dsa = _dsa()
    cfg_big, inp, idx = _case(256, lk, k, seed=lk + k)
    p_big = dsa.make_problem(cfg_big, out_dtype="f32")
    p_small = dsa.make_problem(C.scaled(cfg_big, batch=2), out_dtype="f32")
    assert dsa.attn_splits(p_big) == 1 and dsa.attn_splits(p_small) > 1
    lse_b = torch.empty(256, 1, 128, dtype=torch.float32, device=DEV)
    out_b, lse_b = dsa.sparse_mla_attn(p_big, inp["q_attn"], inp["kv"], idx, lse=lse_b)
    lse_s = torch.empty(2, 1, 128, dtype=torch.float32, device=DEV)
    out_s, lse_s = dsa.sparse_mla_attn(p_small, inp["q_attn"][:2].contiguous(), inp["kv"][:2].contiguous(),
                                       idx[:2].contiguous(), lse=lse_s)
    torch.cuda.synchronize()
    for b in range(2):
        vmax = inp["kv"][b, idx[b, 0].long(), :512].float().abs().max().item()
        diff = (out_s[b] - out_b[b]).abs().max().item()
        assert diff <= 2.0 ** -8 * vmax, (b, diff, vmax)
    np.testing.assert_allclose(lse_s.cpu().numpy(), lse_b[:2].cpu().numpy(), rtol=1e-5, atol=1e-5)


# two rows split 16, 32 (4096 keys), 4 or 2 ways
@pytest.mark.parametrize("lk,k", [(4096, 2048), (20000, 2048), (9000, 4096), (3000, 512), (3000, 300)])
def test_split_merge_bf16_output_within_double_rounding_of_fp32(lk, k):
    """Same launch plan, two output types.  The fp32 output merges fp32
    partials; the bf16 one merges bf16-rounded partials O_s (each off by at
    most 2^-9 |O_s| <= 2^-9 max|v|, and the merge weights sum to 1) and then
    rounds once more (2^-9 |out|).  So the two differ by at most
    2^-8 * max|v| over the chosen rows, and the LSEs, which never pass
    through bf16, are bit-identical."""
    dsa = _dsa()
    cfg, inp, idx = _case(2, lk, k, seed=lk * 3 + k)
    p32 = dsa.make_problem(cfg, out_dtype="f32")
    p16 = dsa.make_problem(cfg, out_dtype="bf16")
    assert dsa.attn_splits(p32) > 1 and dsa.attn_splits(p16) == dsa.attn_splits(p32)
    l32 = torch.empty(2, 1, 128, dtype=torch.float32, device=DEV)
    l16 = torch.empty(2, 1, 128, dtype=torch.float32, device=DEV)
    o32, l32 = dsa.sparse_mla_attn(p32, inp["q_attn"], inp["kv"], idx, lse=l32)
    o16, l16 = dsa.sparse_mla_attn(p16, inp["q_attn"], inp["kv"], idx, lse=l16)
    torch.cuda.synchronize()
    for b in range(2):
        vmax = inp["kv"][b, idx[b, 0].long(), :512].float().abs().max().item()
        diff = (o16[b].float() - o32[b]).abs().max().item()
        assert diff <= 2.0 ** -8 * vmax, (b, diff, vmax)
    assert torch.equal(l16, l32)


def test_split_merge_is_bit_reproducible():
    dsa = _dsa()
    cfg, inp, idx = _case(3, 20000, 2048, seed=7)
    p = dsa.make_problem(cfg)
    assert dsa.attn_splits(p) > 1
    outs = []
    for _ in range(6):
        o, _ = dsa.sparse_mla_attn(p, inp["q_attn"], inp["kv"], idx)
        outs.append(o.view(torch.uint8).clone())
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
