"""MI355X (gfx950) DeepSeek Sparse Attention hot path: indexer scores,
exact top-k and sparse MLA attention, behind the C ABI in include/dsa.h.

The Python layer only marshals torch tensors to the library; see dsa.py.
"""
from .dsa import (  # noqa: F401
    DSAError, Problem, StageEvents, abi_version, attn_splits, cache_append, topk_slice_len, topk_list_slots, forward, forward_chunks, forward_static,
    index_rotate_quantize, index_q_proj, head_weights_proj, head_weights_workspace_size, out_unabsorb,
    index_scores, lib,
    make_problem, sparse_mla_attn, status_string, topk, workspace_size,
    DSA_OP_ATTN, DSA_OP_FORWARD, DSA_OP_TOPK, DSA_NUM_STAGES, STAGE_NAMES, DSA_F32, DSA_BF16, DSA_FP8_E4M3,
    DSA_ERR_EXCEEDS_SCRATCH, DSA_STATIC_SCRATCH_BYTES,
)
