"""The five synthetic DSA workloads, as shape/dtype/seed records.

Dimensions at V3.2 size come from the released configuration excerpt on the
atlas "DeepSeek-V3.2-Exp" token-ids page (config_671B_v3.2: n_heads 128,
kv_lora_rank 512, qk_nope_head_dim 128, qk_rope_head_dim 64, index_n_heads 64,
index_head_dim 128, index_topk 2048, scale_fmt ue8m0).  The workload shapes
themselves (batch, lengths, distributions, planting) are the five synthetic
configurations this library is measured on; the pages print no workload.

This module holds no arithmetic of the method: it only names shapes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, asdict


@dataclass(frozen=True)
class DSAConfig:
    name: str
    batch: int          # B sequences
    q_len: int          # Lq queries per sequence (query i sits at position kv_len - q_len + i)
    kv_len: int         # Lk cached tokens per sequence
    index_heads: int    # H
    index_dim: int      # D
    topk: int           # K
    attn_heads: int     # NH
    qk_dim: int         # Dqk = latent + rope
    v_dim: int          # Dv = latent (values are the leading Dv dims of each kv row)
    softmax_scale: float
    index_dtype: str    # "f32" | "bf16" | "fp8_e4m3"
    attn_dtype: str     # "f32" | "bf16"
    seed: int
    planting: str       # "per_query" | "fraction" | "stratified" | "none"
    plant_count: int = 0
    description: str = ""

    @property
    def n_queries(self) -> int:
        return self.batch * self.q_len

    def visible(self, i: int) -> int:
        """Number of keys query i sees: positions 0..p inclusive, p = Lk - Lq + i."""
        return self.kv_len - self.q_len + i + 1

    def as_dict(self) -> dict:
        return asdict(self)


TINY = DSAConfig(
    name="tiny_prefill_f32_L256", batch=1, q_len=256, kv_len=256,
    index_heads=4, index_dim=32, topk=16,
    attn_heads=8, qk_dim=80, v_dim=64, softmax_scale=1.0 / math.sqrt(80.0),
    index_dtype="f32", attn_dtype="f32", seed=1501,
    planting="per_query", plant_count=4,
    description="tiny causal prefill, fp32, 4 planted earlier keys per query")

DECODE_32K = DSAConfig(
    name="decode_bf16_B32_ctx32768", batch=32, q_len=1, kv_len=32768,
    index_heads=64, index_dim=128, topk=2048,
    attn_heads=128, qk_dim=576, v_dim=512, softmax_scale=1.0 / math.sqrt(192.0),
    index_dtype="bf16", attn_dtype="bf16", seed=1502,
    planting="fraction", plant_count=328,
    description="decode, 32 sequences x 1 query at context 32768, 1% planted keys")

PREFILL_8K = DSAConfig(
    name="prefill_bf16_L8192", batch=1, q_len=8192, kv_len=8192,
    index_heads=64, index_dim=128, topk=2048,
    attn_heads=128, qk_dim=576, v_dim=512, softmax_scale=1.0 / math.sqrt(192.0),
    index_dtype="bf16", attn_dtype="bf16", seed=1503,
    planting="none",
    description="causal prefill, one sequence of 8192 tokens")

DECODE_128K = DSAConfig(
    name="decode_bf16_B8_ctx131072", batch=8, q_len=1, kv_len=131072,
    index_heads=64, index_dim=128, topk=2048,
    attn_heads=128, qk_dim=576, v_dim=512, softmax_scale=1.0 / math.sqrt(192.0),
    index_dtype="bf16", attn_dtype="bf16", seed=1504,
    planting="stratified", plant_count=64,
    description="long-context decode, 8 sequences x 1 query at context 131072, 64 stratified planted keys")

PREFILL_64K_FP8 = DSAConfig(
    name="prefill_fp8idx_L65536", batch=1, q_len=65536, kv_len=65536,
    index_heads=64, index_dim=128, topk=2048,
    attn_heads=128, qk_dim=576, v_dim=512, softmax_scale=1.0 / math.sqrt(192.0),
    index_dtype="fp8_e4m3", attn_dtype="bf16", seed=1505,
    planting="none",
    description="long causal prefill, fp8 E4M3 indexer with per-row ue8m0 scales, bf16 MLA")

CONFIGS = [TINY, DECODE_32K, PREFILL_8K, DECODE_128K, PREFILL_64K_FP8]
BY_NAME = {c.name: c for c in CONFIGS}


def scaled(cfg: DSAConfig, **changes) -> DSAConfig:
    """A copy of cfg with some fields replaced (used for reduced-size parity cases)."""
    d = cfg.as_dict()
    d.update(changes)
    return DSAConfig(**d)
