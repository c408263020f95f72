"""Plain, slow, fp64 CPU oracle of the DeepSeek Sparse Attention (DSA) hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the bench's cpu_baseline leg may import or run this module; the library's
product path never calls it and shares no code with it.

What it computes, step by step, and where each step comes from:

  1. Index scores (lightning indexer).  The HF model doc "DeepSeek-V3.2",
     section "DeepSeek Sparse Attention (DSA)", item 1, describes a light
     scorer with few heads that gives each query a score against every key
     before it; the paragraph after the list says the index keys are a single
     head of index_head_dim per token; the altools.ai page, "Technical
     Principles", says the scorer uses a small number of index heads; the
     usage example keeps an indexer `weights_proj` (per-query head weights).
     The pages never print the formula.  Reading used here: per head a dot
     product q_h . k_s, a ReLU gate, a per-query head weight w_h, summed over
     heads:  I[s] = sum_h w_h * max(0, q_h . k_s).
  2. Causal candidate set.  The same item scores a query against the keys
     before it; together with the causal mask of the atlas "DeepSeek-V3.2-Exp" transformer-forward excerpt,
     which blanks only strictly-upper entries (triu with offset 1): query at
     position p sees keys 0..p, itself included.  Decode (one query) uses no
     mask, so the single query at p = Lk-1 sees the whole cache.
  3. Top-k.  Item 2 of the same DSA section: each query keeps the index_topk
     best-scoring tokens (2048 by default; the visual-learn page, "Different
     questions select different tokens", makes that number a ceiling).  Reading:
     K' = min(K, n); order by (score descending, position ascending); report
     the chosen positions ascending, padded with -1.
  4. Sparse attention.  Item 2 again: main MLA attention runs only over the
     chosen tokens, expressed as an additive mask; the altools.ai page says
     MLA runs in MQA form with key entries shared by all query heads; the
     visual-learn page says the cached entries are MLA's compressed vectors.
     Absorbed form: each kv row is latent (kv_lora_rank) + rope dims; values
     are its leading Dv (= latent) dims; softmax scale given by the caller.

Pins (tests marked "not gpu"): hand-worked score/select/attention fixtures in
tests/golden, invariants (head permutation, positive weight scaling,
orthonormal Hadamard rotation of q and k, causality), brute-force top-k,
K >= n equal to dense causal attention (a separately written masked dense
routine and torch's scaled_dot_product_attention in fp64), K = 1 and equal
logits closed forms, logsumexp vs scipy, E4M3 decode vs torch's float8 type.
Parity unpinned: the head-combination formula of step 1 (the pages never
print it; the reading above is fixed by the workload description only).
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


# --------------------------------------------------------------------------
# FP8 E4M3 (OCP "fn" variant) decode, written from the format's definition:
# 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
# gives subnormals m/8 * 2^-6; bit pattern S.1111.111 is NaN; no infinities.
# ue8m0 scale byte e encodes 2^(e-127) (the "scale_fmt: ue8m0" entry of the
# released configuration excerpt on the atlas token-ids page).
# --------------------------------------------------------------------------
def e4m3_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.power(2.0, e - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal) * sign
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return val.astype(np.float64)


def ue8m0_decode(exps) -> np.ndarray:
    return np.power(2.0, np.asarray(exps, dtype=np.float64) - 127.0)


def dequant_rows(codes, exps) -> np.ndarray:
    """codes [..., D] uint8 E4M3, exps [...] uint8 ue8m0 -> fp64 values."""
    return e4m3_decode(codes) * ue8m0_decode(exps)[..., None]


# --------------------------------------------------------------------------
# Step 1-2: index scores
# --------------------------------------------------------------------------
def visible_count(q_len: int, kv_len: int, i: int) -> int:
    """Keys seen by query i: positions 0..p with p = kv_len - q_len + i."""
    return kv_len - q_len + i + 1


def index_scores_row(q_i: np.ndarray, k: np.ndarray, w_i: np.ndarray, n: int) -> np.ndarray:
    """Scores of one query against keys 0..n-1.

    q_i [H, D], k [Lk, D], w_i [H] (fp64).  Returns [n] fp64:
    I[s] = sum_h w_h * max(0, q_h . k_s), heads summed in index order.
    """
    x = q_i @ k[:n].T                    # [H, n] per-head dot products
    gated = np.maximum(x, 0.0)           # ReLU gate
    acc = np.zeros(n, dtype=np.float64)
    for h in range(q_i.shape[0]):
        acc += w_i[h] * gated[h]
    return acc


def index_scores(q_idx, k_idx, head_w, q_len: int, kv_len: int) -> np.ndarray:
    """q_idx [B,Lq,H,D], k_idx [B,Lk,D], head_w [B,Lq,H] -> scores [B,Lq,Lk] fp64.

    Entries beyond a query's causal limit are -inf.
    """
    q_idx = np.asarray(q_idx, dtype=np.float64)
    k_idx = np.asarray(k_idx, dtype=np.float64)
    head_w = np.asarray(head_w, dtype=np.float64)
    B = q_idx.shape[0]
    out = np.full((B, q_len, kv_len), NEG_INF, dtype=np.float64)
    for b in range(B):
        for i in range(q_len):
            n = visible_count(q_len, kv_len, i)
            out[b, i, :n] = index_scores_row(q_idx[b, i], k_idx[b], head_w[b, i], n)
    return out


# --------------------------------------------------------------------------
# Step 3: top-k selection
# --------------------------------------------------------------------------
def topk_row(row, n: int, k: int) -> np.ndarray:
    """Positions of the K' = min(k, n) best entries of row[:n].

    Order: higher score first, lower position first among equal scores
    (+0.0 and -0.0 compare equal).  Returned ascending, padded with -1 to k.
    """
    row = np.asarray(row)
    kk = min(k, n)
    out = np.full(k, -1, dtype=np.int64)
    if kk == n:
        out[:n] = np.arange(n)
        return out
    pos = np.arange(n)
    order = np.lexsort((pos, -row[:n].astype(np.float64)))   # last key is primary
    out[:kk] = np.sort(order[:kk])
    return out


def topk(scores, q_len: int, kv_len: int, k: int) -> np.ndarray:
    """scores [B,Lq,Lk] -> indices [B,Lq,k] int64 (ascending, -1 padded)."""
    scores = np.asarray(scores)
    B = scores.shape[0]
    out = np.full((B, q_len, k), -1, dtype=np.int64)
    for b in range(B):
        for i in range(q_len):
            out[b, i] = topk_row(scores[b, i], visible_count(q_len, kv_len, i), k)
    return out


# --------------------------------------------------------------------------
# Step 4: sparse MLA attention (absorbed, MQA: one kv row shared by all heads)
# --------------------------------------------------------------------------
def sparse_attention_row(qa_i: np.ndarray, kv: np.ndarray, sel: np.ndarray, scale: float, v_dim: int):
    """One query.  qa_i [NH, Dqk], kv [Lk, Dqk], sel: chosen positions (-1 ignored).

    Returns (out [NH, Dv], lse [NH]) in fp64, softmax over the chosen rows only.
    """
    s = np.asarray([j for j in sel if j >= 0], dtype=np.int64)
    rows = kv[s]                                   # [K', Dqk]
    z = scale * (qa_i @ rows.T)                    # [NH, K'] logits
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e @ rows[:, :v_dim]) / l                # values: leading Dv dims
    lse = m[:, 0] + np.log(l[:, 0])
    return out, lse


def sparse_attention(q_attn, kv, topk_idx, scale: float, v_dim: int):
    """q_attn [B,Lq,NH,Dqk], kv [B,Lk,Dqk], topk_idx [B,Lq,K] -> (out [B,Lq,NH,Dv], lse [B,Lq,NH])."""
    q_attn = np.asarray(q_attn, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    B, Lq, NH, _ = q_attn.shape
    out = np.zeros((B, Lq, NH, v_dim), dtype=np.float64)
    lse = np.zeros((B, Lq, NH), dtype=np.float64)
    for b in range(B):
        for i in range(Lq):
            out[b, i], lse[b, i] = sparse_attention_row(q_attn[b, i], kv[b], topk_idx[b, i], scale, v_dim)
    return out, lse


def dense_masked_attention(q_attn, kv, topk_idx, q_len: int, kv_len: int, scale: float, v_dim: int):
    """Brute force: ordinary softmax attention over ALL kv_len keys with an
    additive mask that is 0 on (causally visible AND selected) keys and -inf
    elsewhere.  Written separately from sparse_attention as its check.
    """
    q_attn = np.asarray(q_attn, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    B, Lq, NH, _ = q_attn.shape
    out = np.zeros((B, Lq, NH, v_dim), dtype=np.float64)
    lse = np.zeros((B, Lq, NH), dtype=np.float64)
    for b in range(B):
        for i in range(Lq):
            p = kv_len - q_len + i
            mask = np.full(kv_len, NEG_INF)
            for j in topk_idx[b, i]:
                if 0 <= j <= p:
                    mask[j] = 0.0
            z = scale * (q_attn[b, i] @ kv[b].T) + mask[None, :]
            m = np.max(z, axis=1, keepdims=True)
            e = np.exp(z - m)
            l = np.sum(e, axis=1, keepdims=True)
            out[b, i] = (e @ kv[b][:, :v_dim]) / l
            lse[b, i] = m[:, 0] + np.log(l[:, 0])
    return out, lse


# --------------------------------------------------------------------------
# Whole path
# --------------------------------------------------------------------------
def as_f64_index_inputs(q_idx, q_scale, k_idx, k_scale):
    """Index q/k as fp64 values; fp8 inputs are decoded with their row scales."""
    if q_scale is not None:
        return dequant_rows(q_idx, q_scale), dequant_rows(k_idx, k_scale)
    return np.asarray(q_idx, dtype=np.float64), np.asarray(k_idx, dtype=np.float64)


def forward(q_idx, q_scale, k_idx, k_scale, head_w, q_attn, kv, topk_k: int, scale: float, v_dim: int):
    """Scores -> top-k -> sparse attention for every query.  Arrays are numpy.

    Returns dict(scores [B,Lq,Lk] fp64, topk [B,Lq,K] int64, out [B,Lq,NH,Dv], lse [B,Lq,NH]).
    """
    qf, kf = as_f64_index_inputs(q_idx, q_scale, k_idx, k_scale)
    q_len, kv_len = qf.shape[1], kf.shape[1]
    sc = index_scores(qf, kf, head_w, q_len, kv_len)
    idx = topk(sc, q_len, kv_len, topk_k)
    out, lse = sparse_attention(q_attn, kv, idx, scale, v_dim)
    return dict(scores=sc, topk=idx, out=out, lse=lse)


def forward_rows(q_idx, q_scale, k_idx, k_scale, head_w, q_attn, kv, rows, q_len: int,
                 topk_k: int, scale: float, v_dim: int, kv_len: int | None = None):
    """The whole path for a chosen list of (b, i) query rows only.

    q_idx/head_w/q_attn are indexed [b, i]; k_idx/kv are the caches
    [B, >= Lk, ...].  kv_len is the context Lk (default: the caches' length);
    cache slots at or beyond it are never read.  Returns a list of dicts
    (scores [n], topk [K], out, lse), the same values forward() gives for
    those rows.
    """
    res = []
    for (b, i) in rows:
        if q_scale is not None:
            qi = dequant_rows(q_idx[b, i], q_scale[b, i])
            kb = dequant_rows(k_idx[b], k_scale[b])
        else:
            qi = np.asarray(q_idx[b, i], dtype=np.float64)
            kb = np.asarray(k_idx[b], dtype=np.float64)
        Lk = kb.shape[0] if kv_len is None else kv_len
        n = visible_count(q_len, Lk, i)
        sc = index_scores_row(qi, kb, np.asarray(head_w[b, i], dtype=np.float64), n)
        sel = topk_row(sc, n, topk_k)
        o, l = sparse_attention_row(np.asarray(q_attn[b, i], dtype=np.float64),
                                    np.asarray(kv[b], dtype=np.float64), sel, scale, v_dim)
        res.append(dict(scores=sc, topk=sel, out=o, lse=l))
    return res


def topk_band_check(oracle_scores_row: np.ndarray, gpu_sel, n: int, k: int, rel_eps: float = 1e-6):
    """Accept a selected set against oracle scores, allowing swaps inside a band.

    tau = the oracle's K'-th largest score, eps = rel_eps * max|I| over the row.
    The set must have exactly K' valid entries, contain every s with
    I[s] > tau + eps and no s with I[s] < tau - eps.  Returns (ok, n_swaps,
    message); n_swaps counts chosen positions that differ from the oracle's.
    """
    kk = min(k, n)
    row = np.asarray(oracle_scores_row[:n], dtype=np.float64)
    sel = np.asarray([j for j in gpu_sel if j >= 0], dtype=np.int64)
    if sel.size != kk:
        return False, -1, f"selected {sel.size} positions, expected {kk}"
    if len(np.unique(sel)) != sel.size or (sel.size and (sel.min() < 0 or sel.max() >= n)):
        return False, -1, "duplicate or out-of-range positions"
    if kk == n:
        return True, 0, ""
    tau = np.sort(row)[::-1][kk - 1]
    eps = rel_eps * float(np.max(np.abs(row)))
    chosen = np.zeros(n, dtype=bool)
    chosen[sel] = True
    must = row > tau + eps
    never = row < tau - eps
    if np.any(must & ~chosen):
        return False, -1, f"missing {int(np.sum(must & ~chosen))} positions above the band"
    if np.any(never & chosen):
        return False, -1, f"{int(np.sum(never & chosen))} chosen positions below the band"
    ref = topk_row(row, n, k)
    swaps = int(kk - np.intersect1d(ref[ref >= 0], sel).size)
    return True, swaps, ""
