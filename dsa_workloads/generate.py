"""Seeded synthetic inputs for the DSA workloads.

Both sides of every parity check (the HIP library and the CPU oracle) are fed
from these tensors; the oracle receives host copies of exactly the values the
GPU receives.  Nothing here computes any part of the method: the module draws
normal variates, plants correlated keys into the index-key cache, rounds to
the storage dtype and, for the FP8 workload, encodes rows as E4M3 codes with
one power-of-two (ue8m0) scale per 128-element row.

Recipe (per tensor, each from its own counter-seeded torch.Generator):
  q_idx [B,Lq,H,D], k_idx [B,Lk,D]      ~ N(0,1)
  head_w [B,Lq,H]                        ~ N(0, 1/H)            (fp32 always)
  q_attn [B,Lq,NH,Dqk], kv [B,Lk,Dqk]    ~ N(0,1)
Planting (index keys only): key s <- u_hat + 0.1 z with z ~ N(0,1), where
u_hat = (sum_h w_h q_h) rescaled to norm sqrt(D) is the query's combined
indexer direction; "per_query": for every query position t, min(count, t)
distinct earlier positions (later queries overwrite); "fraction": `count`
distinct positions before the query; "stratified": one position drawn
uniformly in each of `count` equal strata of [0, p-1].
Storage rounding happens once, after planting: bf16 by round-to-nearest-even,
fp8 by the E4M3 encoder below.
"""
from __future__ import annotations

import math
import zlib

import torch

from .configs import DSAConfig

_CHUNK = 1 << 26  # elements per generation chunk (bounds temporary memory)


def _seed(*parts) -> int:
    return zlib.crc32(repr(parts).encode()) & 0x7FFFFFFF


def _normal(shape, seed: int, device, std: float = 1.0) -> torch.Tensor:
    """fp32 N(0, std^2) of the given shape, drawn in fixed-size chunks."""
    numel = 1
    for s in shape:
        numel *= s
    out = torch.empty(numel, dtype=torch.float32, device=device)
    for c, start in enumerate(range(0, numel, _CHUNK)):
        n = min(_CHUNK, numel - start)
        g = torch.Generator(device=device)
        g.manual_seed(_seed(seed, c))
        out[start:start + n] = torch.randn(n, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        out.mul_(std)
    return out.view(*shape)


def _normal_stored(shape, seed: int, device, dtype) -> torch.Tensor:
    """N(0,1) rounded to `dtype`, generated chunk by chunk (no full fp32 copy)."""
    numel = 1
    for s in shape:
        numel *= s
    out = torch.empty(numel, dtype=dtype, device=device)
    for c, start in enumerate(range(0, numel, _CHUNK)):
        n = min(_CHUNK, numel - start)
        g = torch.Generator(device=device)
        g.manual_seed(_seed(seed, c))
        out[start:start + n] = torch.randn(n, generator=g, device=device, dtype=torch.float32).to(dtype)
    return out.view(*shape)


E4M3_MAX = 448.0


def quantize_e4m3_rows(x: torch.Tensor):
    """Encode the last dim of x as OCP E4M3 codes with one ue8m0 scale per row.

    scale = 2^(e-127) with e = 127 + ceil(log2(amax/448)) (e = 127 for an
    all-zero row), codes = RNE(x / scale) (never saturates: |x/scale| <= 448).
    Returns (codes uint8 [..., D], exps uint8 [...]).
    """
    amax = x.abs().amax(dim=-1).to(torch.float64)
    ratio = amax / E4M3_MAX
    e = torch.where(amax > 0, torch.ceil(torch.log2(torch.where(amax > 0, ratio, torch.ones_like(ratio)))),
                    torch.zeros_like(ratio))
    # guard against log2 rounding: make sure amax / 2^e <= 448 and amax / 2^(e-1) > 448
    e = torch.where((amax > 0) & (amax / torch.exp2(e) > E4M3_MAX), e + 1, e)
    e = torch.where((amax > 0) & (amax / torch.exp2(e - 1) <= E4M3_MAX), e - 1, e)
    e = e.clamp(-127, 127)
    scale = torch.exp2(e).to(torch.float32)
    codes = (x / scale.unsqueeze(-1)).to(torch.float8_e4m3fn).view(torch.uint8)
    exps = (e + 127).to(torch.uint8)
    return codes, exps


def _plant_direction(q_row: torch.Tensor, w_row: torch.Tensor, D: int, dev) -> torch.Tensor:
    """u_hat = (sum_h w_h q_h) rescaled to norm sqrt(D), in fp32 on `dev`."""
    u = (w_row.to(torch.float32).unsqueeze(-1) * q_row.to(torch.float32)).sum(0)
    return u * (math.sqrt(D) / torch.clamp(u.norm(), min=1e-30))


def plant_positions(cfg: DSAConfig, b: int, set_index: int = 0):
    """Planted positions per query of sequence b: list (len Lq) of int lists."""
    g = torch.Generator()
    out = []
    for i in range(cfg.q_len):
        p = cfg.kv_len - cfg.q_len + i
        g.manual_seed(_seed(cfg.seed, set_index, "plant", b, i))
        if cfg.planting == "per_query":
            k = min(cfg.plant_count, p)
            pos = torch.randperm(p, generator=g)[:k].tolist() if k > 0 else []
        elif cfg.planting == "fraction":
            pos = torch.randperm(p, generator=g)[:cfg.plant_count].tolist()
        elif cfg.planting == "stratified":
            n = cfg.plant_count
            pos = []
            for j in range(n):
                lo = (j * p) // n
                hi = max(lo + 1, ((j + 1) * p) // n)
                pos.append(lo + int(torch.randint(hi - lo, (1,), generator=g)))
        else:
            pos = []
        out.append(pos)
    return out


def generate(cfg: DSAConfig, device="cpu", set_index: int = 0) -> dict:
    """All inputs of one DSA call for `cfg`, on `device`.

    Keys of the returned dict: q_idx, q_scale, k_idx, k_scale, head_w,
    q_attn, kv, planted.  fp8 index tensors are uint8 E4M3 codes with uint8
    ue8m0 exponents in q_scale [B,Lq,H] / k_scale [B,Lk]; otherwise the
    scales are None.
    """
    B, Lq, Lk = cfg.batch, cfg.q_len, cfg.kv_len
    H, D = cfg.index_heads, cfg.index_dim
    s = (cfg.seed, set_index)
    q = _normal((B, Lq, H, D), _seed(*s, "q_idx"), device)
    k = _normal((B, Lk, D), _seed(*s, "k_idx"), device)
    w = _normal((B, Lq, H), _seed(*s, "head_w"), device, std=1.0 / math.sqrt(H))

    if cfg.index_dtype == "bf16":
        q = q.to(torch.bfloat16)
    planted = []
    if cfg.planting != "none":
        for b in range(B):
            per_q = plant_positions(cfg, b, set_index)
            planted.append(per_q)
            for i, pos in enumerate(per_q):
                if not pos:
                    continue
                u = _plant_direction(q[b, i], w[b, i], D, device)
                z = _normal((len(pos), D), _seed(*s, "plant_noise", b, i), device)
                idx = torch.tensor(pos, dtype=torch.long, device=device)
                k[b].index_copy_(0, idx, u.unsqueeze(0) + 0.1 * z)

    q_scale = k_scale = None
    if cfg.index_dtype == "f32":
        pass
    elif cfg.index_dtype == "bf16":
        k = k.to(torch.bfloat16)
    elif cfg.index_dtype == "fp8_e4m3":
        q, q_scale = quantize_e4m3_rows(q)
        k, k_scale = quantize_e4m3_rows(k)
    else:
        raise ValueError(cfg.index_dtype)

    adt = torch.float32 if cfg.attn_dtype == "f32" else torch.bfloat16
    qa = _normal_stored((B, Lq, cfg.attn_heads, cfg.qk_dim), _seed(*s, "q_attn"), device, adt)
    kv = _normal_stored((B, Lk, cfg.qk_dim), _seed(*s, "kv"), device, adt)
    return dict(q_idx=q.contiguous(), q_scale=q_scale, k_idx=k.contiguous(), k_scale=k_scale,
                head_w=w.contiguous(), q_attn=qa, kv=kv, planted=planted)


def random_score_rows(n_rows: int, row_len: int, seed: int, device="cpu",
                      tie_fraction: float = 0.0, neg_zero: bool = False) -> torch.Tensor:
    """fp32 rows for exercising a top-k selector on its own.

    Values ~ N(0, 8^2); with tie_fraction > 0 a share of entries is copied from
    a few pivot values (exact duplicates), and with neg_zero some entries are
    set to +0.0 and some to -0.0.
    """
    x = _normal((n_rows, row_len), _seed(seed, "rows"), device, std=8.0)
    if tie_fraction > 0:
        g = torch.Generator(device=device)
        g.manual_seed(_seed(seed, "ties"))
        mask = torch.rand(n_rows, row_len, generator=g, device=device) < tie_fraction
        pick = torch.randint(0, 4, (n_rows, row_len), generator=g, device=device)
        pivots = torch.quantile(x.to(torch.float64).cpu(), torch.tensor([0.5, 0.9, 0.95, 0.99], dtype=torch.float64),
                                dim=1).T.to(torch.float32).to(device)
        x = torch.where(mask, torch.gather(pivots, 1, pick), x)
    if neg_zero:
        g = torch.Generator(device=device)
        g.manual_seed(_seed(seed, "zeros"))
        r = torch.rand(n_rows, row_len, generator=g, device=device)
        x = torch.where(r < 0.05, torch.zeros_like(x), x)
        x = torch.where((r >= 0.05) & (r < 0.10), torch.full_like(x, -0.0), x)
    return x.contiguous()


# Sizes of the projections in the released configuration excerpt.
Q_LORA_RANK, HIDDEN, V_HEAD_DIM = 1536, 7168, 128


def generate_projection_inputs(cfg: DSAConfig, device="cpu", set_index: int = 0, q_lora_rank: int = Q_LORA_RANK,
                               hidden: int = HIDDEN, v_head_dim: int = V_HEAD_DIM) -> dict:
    """Seeded bf16 inputs of the projections on either side of the path.

      cq     [B,Lq,R]        ~ N(0,1)      query latent
      wq_b   [H*D, R]        ~ N(0, 1/R)   (index queries come out ~ N(0,1))
      x      [B,Lq,hidden]   ~ N(0,1)      hidden state
      w_proj [H, hidden]     ~ N(0, 1/(hidden*H))   (head weights ~ N(0, 1/H))
      o_lat  [B,Lq,NH,Dv]    ~ N(0,1)      latent attention output
      w_uv   [NH, V, Dv]     ~ N(0, 1/Dv)
    """
    B, Lq, H, D = cfg.batch, cfg.q_len, cfg.index_heads, cfg.index_dim
    NH, Dv = cfg.attn_heads, cfg.v_dim
    s = (cfg.seed, set_index, "proj")
    bf = torch.bfloat16
    return dict(
        cq=_normal_stored((B, Lq, q_lora_rank), _seed(*s, "cq"), device, bf),
        wq_b=_normal((H * D, q_lora_rank), _seed(*s, "wq_b"), device, std=1.0 / math.sqrt(q_lora_rank)).to(bf),
        x=_normal_stored((B, Lq, hidden), _seed(*s, "x"), device, bf),
        w_proj=_normal((H, hidden), _seed(*s, "w_proj"), device, std=1.0 / math.sqrt(hidden * H)).to(bf),
        o_lat=_normal_stored((B, Lq, NH, Dv), _seed(*s, "o_lat"), device, bf),
        w_uv=_normal((NH, v_head_dim, Dv), _seed(*s, "w_uv"), device, std=1.0 / math.sqrt(Dv)).to(bf),
    )
