"""Thin Python binding of libdsa.so (ctypes).

Argument marshalling only: every function checks tensor device, dtype, shape
and contiguity, then passes raw device pointers and torch's current HIP
stream to the C ABI declared in include/dsa.h.  All arithmetic runs in the
library's HIP kernels; there is no fallback.  torch provides device memory
and streams.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_OK, DSA_ERR_INVALID_ARGUMENT, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE_TOO_SMALL, DSA_ERR_HIP, \
    DSA_ERR_EXCEEDS_SCRATCH = range(6)
DSA_STATIC_SCRATCH_BYTES = 96 << 20
DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
DSA_OP_ATTN, DSA_OP_FORWARD, DSA_OP_TOPK = 1, 2, 3
DSA_NUM_STAGES = 4
STAGE_NAMES = ("indexer", "topk", "attention", "combine")

_DTYPE_CODE = {"f32": DSA_F32, "bf16": DSA_BF16, "fp8_e4m3": DSA_FP8_E4M3}


class DSAError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("kv_len", ctypes.c_int32),
        ("index_heads", ctypes.c_int32), ("index_dim", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("attn_heads", ctypes.c_int32), ("qk_dim", ctypes.c_int32), ("v_dim", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("index_dtype", ctypes.c_int), ("attn_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
        ("kv_capacity", ctypes.c_int32),
    ]


_lib = None
_hip = None


def lib() -> ctypes.CDLL:
    """Load libdsa.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m sparse_attention_15_amd.build` "
                           "or __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    P, V, I32, I64, SZ = ctypes.POINTER(Problem), ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sigs = {
        "dsa_index_scores": [P, V, V, V, V, V, V, V],
        "dsa_topk": [P, V, I64, V, V],
        "dsa_topk_ws": [P, V, I64, V, V, SZ, V],
        "dsa_sparse_mla_attn": [P, V, V, V, V, V, V, SZ, V],
        "dsa_forward": [P, V, V, V, V, V, V, V, V, V, V, V, SZ, V],
        "dsa_forward_timed": [P, V, V, V, V, V, V, V, V, V, V, V, SZ, V, I32, V, V],
        "dsa_forward_static": [P, V, V, V, V, V, V, V, V, V, V, V],
    }
    for name, args in sigs.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.dsa_workspace_size.argtypes = [P, I32]
    L.dsa_workspace_size.restype = SZ
    L.dsa_forward_chunks.argtypes = [P]
    L.dsa_forward_chunks.restype = I32
    L.dsa_forward_attn_splits.argtypes = [P]
    L.dsa_forward_attn_splits.restype = I32
    L.dsa_forward_topk_slice_len.argtypes = [P]
    L.dsa_forward_topk_slice_len.restype = I32
    L.dsa_forward_topk_list_slots.argtypes = [P]
    L.dsa_forward_topk_list_slots.restype = I32
    L.dsa_index_rotate_quantize.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.dsa_index_rotate_quantize.restype = ctypes.c_int
    L.dsa_cache_append.argtypes = [P, ctypes.c_int32] + [ctypes.c_void_p] * 6 + [ctypes.c_void_p]
    L.dsa_cache_append.restype = ctypes.c_int
    for name, extra in (("dsa_index_q_proj", [I32, V, V, V, ctypes.c_int, V]),
                        ("dsa_head_weights_proj", [I32, V, V, V, V, SZ, V]),
                        ("dsa_out_unabsorb", [I32, V, V, V, ctypes.c_int, V])):
        f = getattr(L, name)
        f.argtypes = [P] + extra
        f.restype = ctypes.c_int
    L.dsa_head_weights_workspace_size.argtypes = [P, I32]
    L.dsa_head_weights_workspace_size.restype = SZ
    L.dsa_status_string.argtypes = [ctypes.c_int]
    L.dsa_status_string.restype = ctypes.c_char_p
    L.dsa_abi_version.argtypes = []
    L.dsa_abi_version.restype = I32
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().dsa_status_string(status).decode()


def abi_version() -> int:
    return lib().dsa_abi_version()


@dataclass
class Shape:
    batch: int
    q_len: int
    kv_len: int
    index_heads: int
    index_dim: int
    topk: int
    attn_heads: int
    qk_dim: int
    v_dim: int
    softmax_scale: float
    index_dtype: str
    attn_dtype: str
    out_dtype: str


def make_problem(cfg, out_dtype: str | None = None, kv_capacity: int = 0) -> Problem:
    """Problem from any object with the DSAConfig field names; kv_capacity is
    the caches' tokens per sequence (0: kv_len)."""
    od = out_dtype or cfg.attn_dtype
    return Problem(cfg.batch, cfg.q_len, cfg.kv_len, cfg.index_heads, cfg.index_dim, cfg.topk,
                   cfg.attn_heads, cfg.qk_dim, cfg.v_dim, float(cfg.softmax_scale),
                   _DTYPE_CODE[cfg.index_dtype], _DTYPE_CODE[cfg.attn_dtype], _DTYPE_CODE[od], kv_capacity)


def _cap(p: Problem) -> int:
    return p.kv_capacity if p.kv_capacity else p.kv_len


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


_TORCH_DT = {DSA_F32: torch.float32, DSA_BF16: torch.bfloat16, DSA_FP8_E4M3: torch.uint8}


def _ptr(t, name, dtype=None, shape=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None:
        ok = t.dtype == dtype or (dtype == torch.uint8 and t.dtype == torch.float8_e4m3fn)
        if not ok:
            raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _check(status: int, what: str):
    if status != DSA_OK:
        raise DSAError(status, what)


def _index_args(p: Problem, q_idx, q_scale, k_idx, k_scale, head_w):
    B, Lq, Lk, H, D = p.batch, p.q_len, p.kv_len, p.index_heads, p.index_dim
    it = _TORCH_DT[p.index_dtype]
    fp8 = p.index_dtype == DSA_FP8_E4M3
    return (_ptr(q_idx, "q_idx", it, (B, Lq, H, D)),
            _ptr(q_scale, "q_scale", torch.uint8, (B, Lq, H), allow_none=not fp8),
            _ptr(k_idx, "k_idx", it, (B, _cap(p), D)),
            _ptr(k_scale, "k_scale", torch.uint8, (B, _cap(p)), allow_none=not fp8),
            _ptr(head_w, "head_w", torch.float32, (B, Lq, H)))


def index_scores(p: Problem, q_idx, q_scale, k_idx, k_scale, head_w, scores=None) -> torch.Tensor:
    """[B, Lq, Lk] fp32 scores, -inf beyond each query's causal limit."""
    if scores is None:
        scores = torch.empty(p.batch, p.q_len, p.kv_len, dtype=torch.float32, device=q_idx.device)
    args = _index_args(p, q_idx, q_scale, k_idx, k_scale, head_w)
    sp = _ptr(scores, "scores", torch.float32, (p.batch, p.q_len, p.kv_len))
    _check(lib().dsa_index_scores(ctypes.byref(p), *args, sp, _stream()), "dsa_index_scores")
    return scores


def topk(p: Problem, scores, out=None, workspace=None) -> torch.Tensor:
    """[B, Lq, K] int32 positions (ascending, -1 padded) from fp32 score rows.

    scores: [B, Lq, S] with S >= Lk (row stride S); only the causal prefix is read.
    workspace: None (dsa_topk: one work-group per row), "auto" or a uint8
    device tensor (dsa_topk_ws: few long rows spread over work-groups per slice).
    """
    if scores.dim() != 3 or scores.shape[0] != p.batch or scores.shape[1] != p.q_len:
        raise ValueError(f"scores: shape {tuple(scores.shape)}")
    if out is None:
        out = torch.empty(p.batch, p.q_len, p.topk, dtype=torch.int32, device=scores.device)
    sp = _ptr(scores, "scores", torch.float32)
    op = _ptr(out, "topk_idx", torch.int32, (p.batch, p.q_len, p.topk))
    if workspace is None:
        _check(lib().dsa_topk(ctypes.byref(p), sp, scores.shape[2], op, _stream()), "dsa_topk")
        return out
    ws = _workspace(p, DSA_OP_TOPK, None if isinstance(workspace, str) else workspace, scores.device)
    _check(lib().dsa_topk_ws(ctypes.byref(p), sp, scores.shape[2], op, ctypes.c_void_p(ws.data_ptr()),
                             ws.numel(), _stream()), "dsa_topk_ws")
    return out


def workspace_size(p: Problem, op: int) -> int:
    return int(lib().dsa_workspace_size(ctypes.byref(p), op))


def forward_chunks(p: Problem) -> int:
    return int(lib().dsa_forward_chunks(ctypes.byref(p)))


def attn_splits(p: Problem) -> int:
    return int(lib().dsa_forward_attn_splits(ctypes.byref(p)))


def topk_slice_len(p: Problem) -> int:
    """Positions per work-group of forward's sliced top-k (0: not used)."""
    return int(lib().dsa_forward_topk_slice_len(ctypes.byref(p)))


def topk_list_slots(p: Problem) -> int:
    """List slots per 2048-key chunk of forward's filtered top-k (0: not used)."""
    return int(lib().dsa_forward_topk_list_slots(ctypes.byref(p)))


def cache_append(p: Problem, k_new, k_new_scale, kv_new, k_idx, k_scale, kv):
    """Append n_new tokens per sequence at positions p.kv_len.. of the caches
    (k_new [B, n_new, D], kv_new [B, n_new, Dqk]; caches [B, kv_capacity, ...])."""
    B = p.batch
    n_new = k_new.shape[1]
    it, at = _TORCH_DT[p.index_dtype], _TORCH_DT[p.attn_dtype]
    fp8 = p.index_dtype == DSA_FP8_E4M3
    args = (_ptr(k_new, "k_new", it, (B, n_new, p.index_dim)),
            _ptr(k_new_scale, "k_new_scale", torch.uint8, (B, n_new), allow_none=not fp8),
            _ptr(kv_new, "kv_new", at, (B, n_new, p.qk_dim)),
            _ptr(k_idx, "k_idx", it, (B, _cap(p), p.index_dim)),
            _ptr(k_scale, "k_scale", torch.uint8, (B, _cap(p)), allow_none=not fp8),
            _ptr(kv, "kv", at, (B, _cap(p), p.qk_dim)))
    _check(lib().dsa_cache_append(ctypes.byref(p), n_new, *args, _stream()), "dsa_cache_append")


def index_rotate_quantize(x: torch.Tensor, codes: torch.Tensor = None, scales: torch.Tensor = None):
    """FP8 index vectors from bf16 / f32 activations: x [..., 128] ->
    (codes uint8 [..., 128], scales uint8 [...]); see dsa_index_rotate_quantize."""
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise DSAError(DSA_ERR_INVALID_ARGUMENT, "index_rotate_quantize: x must be bf16 or f32")
    if not x.is_contiguous() or x.shape[-1] != 128 or not x.is_cuda:
        raise DSAError(DSA_ERR_INVALID_ARGUMENT, "index_rotate_quantize: x must be a contiguous CUDA tensor [..., 128]")
    rows = x.numel() // 128
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1], dtype=torch.uint8, device=x.device)
    if codes.dtype != torch.uint8 or codes.numel() != x.numel() or scales.dtype != torch.uint8 or scales.numel() != rows:
        raise DSAError(DSA_ERR_INVALID_ARGUMENT, "index_rotate_quantize: output shapes / dtypes")
    dt = DSA_F32 if x.dtype == torch.float32 else DSA_BF16
    _check(lib().dsa_index_rotate_quantize(ctypes.c_void_p(x.data_ptr()), dt, rows, 128,
                                           ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                                           _stream()), "dsa_index_rotate_quantize")
    return codes, scales


def _proj_out_dtype(dtype) -> int:
    if dtype == torch.bfloat16:
        return DSA_BF16
    if dtype == torch.float32:
        return DSA_F32
    raise DSAError(DSA_ERR_INVALID_ARGUMENT, "projection outputs are bf16 or f32")


def index_q_proj(p: Problem, cq, wq_b, out=None, dtype=torch.bfloat16) -> torch.Tensor:
    """Index query from the query latent: cq [B, Lq, R] bf16, wq_b [H*D, R] bf16
    -> q_idx [B, Lq, H, D]; see dsa_index_q_proj."""
    R = cq.shape[-1]
    if out is None:
        out = torch.empty(p.batch, p.q_len, p.index_heads, p.index_dim, dtype=dtype, device=cq.device)
    args = (_ptr(cq, "cq", torch.bfloat16, (p.batch, p.q_len, R)),
            _ptr(wq_b, "wq_b", torch.bfloat16, (p.index_heads * p.index_dim, R)),
            _ptr(out, "q_idx", out.dtype, (p.batch, p.q_len, p.index_heads, p.index_dim)))
    _check(lib().dsa_index_q_proj(ctypes.byref(p), R, *args, _proj_out_dtype(out.dtype), _stream()),
           "dsa_index_q_proj")
    return out


def head_weights_workspace_size(p: Problem, dim: int) -> int:
    return int(lib().dsa_head_weights_workspace_size(ctypes.byref(p), dim))


def head_weights_proj(p: Problem, x, w_proj, out=None, workspace="auto") -> torch.Tensor:
    """Head weights from the hidden state: x [B, Lq, dim] bf16, w_proj [H, dim]
    bf16 -> head_w [B, Lq, H] fp32; see dsa_head_weights_proj.  workspace:
    "auto" allocates what dsa_head_weights_workspace_size asks for, None
    passes none, or a uint8 CUDA tensor."""
    dim = x.shape[-1]
    if out is None:
        out = torch.empty(p.batch, p.q_len, p.index_heads, dtype=torch.float32, device=x.device)
    args = (_ptr(x, "x", torch.bfloat16, (p.batch, p.q_len, dim)),
            _ptr(w_proj, "w_proj", torch.bfloat16, (p.index_heads, dim)),
            _ptr(out, "head_w", torch.float32, (p.batch, p.q_len, p.index_heads)))
    if isinstance(workspace, str):
        n = head_weights_workspace_size(p, dim)
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device) if n else None
    wsp = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    wsb = workspace.numel() if workspace is not None else 0
    _check(lib().dsa_head_weights_proj(ctypes.byref(p), dim, *args, wsp, wsb, _stream()), "dsa_head_weights_proj")
    return out


def out_unabsorb(p: Problem, o_latent, w_uv, out=None, dtype=torch.bfloat16) -> torch.Tensor:
    """Per-head un-absorption: o_latent [B, Lq, NH, Dv] bf16, w_uv [NH, V, Dv]
    bf16 -> out [B, Lq, NH, V]; see dsa_out_unabsorb."""
    V = w_uv.shape[1]
    if out is None:
        out = torch.empty(p.batch, p.q_len, p.attn_heads, V, dtype=dtype, device=o_latent.device)
    args = (_ptr(o_latent, "o_latent", torch.bfloat16, (p.batch, p.q_len, p.attn_heads, p.v_dim)),
            _ptr(w_uv, "w_uv", torch.bfloat16, (p.attn_heads, V, p.v_dim)),
            _ptr(out, "out", out.dtype, (p.batch, p.q_len, p.attn_heads, V)))
    _check(lib().dsa_out_unabsorb(ctypes.byref(p), V, *args, _proj_out_dtype(out.dtype), _stream()),
           "dsa_out_unabsorb")
    return out


def _out_tensor(p: Problem, device):
    dt = torch.float32 if p.out_dtype == DSA_F32 else torch.bfloat16
    return torch.empty(p.batch, p.q_len, p.attn_heads, p.v_dim, dtype=dt, device=device)


def _attn_args(p: Problem, q_attn, kv, out, lse):
    B, Lq, Lk = p.batch, p.q_len, p.kv_len
    at = _TORCH_DT[p.attn_dtype]
    ot = torch.float32 if p.out_dtype == DSA_F32 else torch.bfloat16
    return (_ptr(q_attn, "q_attn", at, (B, Lq, p.attn_heads, p.qk_dim)),
            _ptr(kv, "kv", at, (B, _cap(p), p.qk_dim)),
            _ptr(out, "out", ot, (B, Lq, p.attn_heads, p.v_dim)),
            _ptr(lse, "lse", torch.float32, (B, Lq, p.attn_heads), allow_none=True))


def _workspace(p: Problem, op: int, workspace, device):
    need = workspace_size(p, op)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    if workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, needs {need}")
    return workspace


def sparse_mla_attn(p: Problem, q_attn, kv, topk_idx, out=None, lse=None, workspace=None):
    """(out [B,Lq,NH,Dv], lse) of attention over the listed positions."""
    if out is None:
        out = _out_tensor(p, q_attn.device)
    qa, kvp, op, lp = _attn_args(p, q_attn, kv, out, lse)
    ip = _ptr(topk_idx, "topk_idx", torch.int32, (p.batch, p.q_len, p.topk))
    ws = _workspace(p, DSA_OP_ATTN, workspace, q_attn.device)
    _check(lib().dsa_sparse_mla_attn(ctypes.byref(p), qa, kvp, ip, op, lp, ctypes.c_void_p(ws.data_ptr()),
                                     ws.numel(), _stream()), "dsa_sparse_mla_attn")
    return out, lse


def forward(p: Problem, q_idx, q_scale, k_idx, k_scale, head_w, q_attn, kv, out=None, lse=None,
            topk_idx=None, workspace=None, events=None, n_events: int = 0):
    """Fused scores -> top-k -> sparse attention.  Returns (out, lse, topk_idx).

    events: optional ctypes array of hipEvent_t (2 per stage slot) for
    per-kernel timing (see hip_events()).
    """
    if out is None:
        out = _out_tensor(p, q_attn.device)
    iargs = _index_args(p, q_idx, q_scale, k_idx, k_scale, head_w)
    qa, kvp, op, lp = _attn_args(p, q_attn, kv, out, lse)
    ip = _ptr(topk_idx, "topk_idx", torch.int32, (p.batch, p.q_len, p.topk), allow_none=True)
    ws = _workspace(p, DSA_OP_FORWARD, workspace, q_attn.device)
    wsp = ctypes.c_void_p(ws.data_ptr())
    if events is None:
        st = lib().dsa_forward(ctypes.byref(p), *iargs, qa, kvp, ip, op, lp, wsp, ws.numel(), _stream())
    else:
        st = lib().dsa_forward_timed(ctypes.byref(p), *iargs, qa, kvp, ip, op, lp, wsp, ws.numel(),
                                     events, n_events, None, _stream())
    _check(st, "dsa_forward")
    return out, lse, topk_idx


def forward_static(p: Problem, q_idx, q_scale, k_idx, k_scale, head_w, q_attn, kv, out=None, lse=None,
                   topk_idx=None):
    """forward() working in the library's static per-GPU scratch instead of a
    workspace (dsa_forward_static: no device allocation inside the call when
    out is given).  Returns (out, lse, topk_idx)."""
    if out is None:
        out = _out_tensor(p, q_attn.device)
    iargs = _index_args(p, q_idx, q_scale, k_idx, k_scale, head_w)
    qa, kvp, op, lp = _attn_args(p, q_attn, kv, out, lse)
    ip = _ptr(topk_idx, "topk_idx", torch.int32, (p.batch, p.q_len, p.topk), allow_none=True)
    _check(lib().dsa_forward_static(ctypes.byref(p), *iargs, qa, kvp, ip, op, lp, _stream()), "dsa_forward_static")
    return out, lse, topk_idx


# ---------------------------------------------------------------- events ---
def _hip_rt():
    """The HIP runtime torch already loaded (same SONAME), for raw events."""
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so.7", mode=ctypes.RTLD_GLOBAL)
        h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        h.hipEventCreate.restype = ctypes.c_int
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventDestroy.restype = ctypes.c_int
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventElapsedTime.restype = ctypes.c_int
        h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        h.hipEventSynchronize.restype = ctypes.c_int
        _hip = h
    return _hip


class StageEvents:
    """2 * n_slots raw hipEvent_t handles for dsa_forward_timed."""

    def __init__(self, n_slots: int):
        h = _hip_rt()
        self.n = 2 * n_slots
        self.arr = (ctypes.c_void_p * self.n)()
        for k in range(self.n):
            ev = ctypes.c_void_p()
            if h.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.arr[k] = ev
        self.n_slots = n_slots

    def elapsed_ms(self, slot: int) -> float:
        h = _hip_rt()
        ms = ctypes.c_float()
        if h.hipEventSynchronize(self.arr[2 * slot + 1]) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        if h.hipEventElapsedTime(ctypes.byref(ms), self.arr[2 * slot], self.arr[2 * slot + 1]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        h = _hip_rt()
        for k in range(self.n):
            if self.arr[k]:
                h.hipEventDestroy(self.arr[k])
                self.arr[k] = None
