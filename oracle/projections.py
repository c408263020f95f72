"""Plain CPU oracle of the projections on either side of the DSA hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the bench's cpu_baseline leg may import or run this module; the library's
product path never calls it and shares no code with it.

What it computes and where it comes from (fp64, numpy matmul as the only
library step):

  1. Index query from the query latent.  The note in the HF model doc
     "DeepSeek-V3.2" (usage notes, on the required query LoRA path): the
     indexer scores queries from the low-rank query latent, through its wq_b
     projection, whose input size is q_lora_rank.  The released configuration
     excerpt on the atlas "DeepSeek-V3.2-Exp" token-ids page gives
     q_lora_rank 1536, index_n_heads 64 and index_head_dim 128.  Reading: a
     plain linear map of the latent to H*D values, head-major (head h owns
     outputs h*D .. h*D + D - 1), weight stored [out][in]:
         q[h, d] = sum_r cq[r] * Wq_b[h*D + d, r].
  2. Head weights from the hidden state.  The usage example of the same doc
     keeps the indexer's weights_proj out of FP8 quantisation (bf16/fp32 in
     the checkpoint); the configuration gives the hidden width dim 7168.
     Reading: a plain linear map to the H head weights, no bias and no extra
     constant (a positive constant would scale every index score of the
     query alike and leave its top-k unchanged):
         w[h] = sum_i x[i] * Wp[h, i].
  3. Un-absorption of the attention output.  The hot path attends in the
     absorbed form (values are the kv_lora_rank = 512 leading latent dims);
     the configuration gives v_head_dim 128 and n_heads 128.  Reading: the
     value half of MLA's key/value up-projection, per head a matrix
     W_UV[a] of shape [v_head_dim][kv_lora_rank]:
         out[a, v] = sum_c O[a, c] * W_UV[a, v, c].
     By linearity this equals attention whose values are the per-head rows
     W_UV[a] kv_j[0:512]; a pin checks exactly that.

The query latent and the hidden state are inputs (the projections and norm
that produce them sit outside this path).
"""
from __future__ import annotations

import numpy as np


def index_q_from_latent(cq: np.ndarray, wq_b: np.ndarray, heads: int, dim: int) -> np.ndarray:
    """cq [..., R], wq_b [heads*dim][R] -> q [..., heads, dim]."""
    cq = np.asarray(cq, dtype=np.float64)
    wq_b = np.asarray(wq_b, dtype=np.float64)
    if wq_b.shape != (heads * dim, cq.shape[-1]):
        raise ValueError("wq_b must be [heads*dim][q_lora_rank]")
    q = cq @ wq_b.T
    return q.reshape(cq.shape[:-1] + (heads, dim))


def head_weights_from_hidden(x: np.ndarray, w_proj: np.ndarray) -> np.ndarray:
    """x [..., dim], w_proj [H][dim] -> w [..., H]."""
    x = np.asarray(x, dtype=np.float64)
    w_proj = np.asarray(w_proj, dtype=np.float64)
    if w_proj.shape[1] != x.shape[-1]:
        raise ValueError("w_proj must be [H][dim]")
    return x @ w_proj.T


def unabsorb_output(o_lat: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """o_lat [..., NH, C], w_uv [NH][V][C] -> out [..., NH, V]."""
    o_lat = np.asarray(o_lat, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    nh, c = o_lat.shape[-2:]
    if w_uv.shape[0] != nh or w_uv.shape[2] != c:
        raise ValueError("w_uv must be [NH][V][C]")
    out = np.empty(o_lat.shape[:-1] + (w_uv.shape[1],))
    for a in range(nh):
        out[..., a, :] = o_lat[..., a, :] @ w_uv[a].T
    return out
