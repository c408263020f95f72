"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the HIP runtime."""
import ctypes
import os
import re

import pytest

from dsa_workloads import configs as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
LIB = os.path.join(ROOT, "sparse_attention_15_amd", "libdsa.so")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:dsa_status_t|size_t|int32_t|const char\*)\s+(dsa_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def dsa():
    if not os.path.exists(LIB):
        pytest.fail("libdsa.so is not built (run __graft_entry__.build())")
    import sparse_attention_15_amd.dsa as d
    return d


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("dsa_index_scores", "dsa_topk", "dsa_sparse_mla_attn", "dsa_forward",
                     "dsa_workspace_size", "dsa_status_string", "dsa_abi_version"):
        assert required in names


def test_library_exports_every_declared_symbol(dsa):
    L = dsa.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
    assert dsa.abi_version() == 6


def test_status_strings(dsa):
    for s in range(6):
        assert dsa.status_string(s)


def _prob(dsa, cfg, **kw):
    p = dsa.make_problem(cfg)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_workspace_size_is_host_only_and_sane(dsa):
    p = dsa.make_problem(C.DECODE_32K)
    ws = dsa.workspace_size(p, dsa.DSA_OP_FORWARD)
    assert ws >= 32 * 32768 * 4 + 32 * 2048 * 4
    assert dsa.workspace_size(p, 99) == 0
    bad = _prob(dsa, C.DECODE_32K, q_len=0)
    assert dsa.workspace_size(bad, dsa.DSA_OP_FORWARD) == 0
    p5 = dsa.make_problem(C.PREFILL_64K_FP8)
    assert dsa.forward_chunks(p5) > 1          # 16 GiB of scores are never materialised at once
    assert dsa.forward_chunks(dsa.make_problem(C.PREFILL_8K)) == 1


def test_attention_split_plan_is_host_only_and_bounded(dsa):
    # decode shapes split each query's list over work-groups until the launch
    # fills the GPU's 256 CUs, with at least 128 keys per split; prefill
    # shapes already have one work-group per query and never split
    assert dsa.attn_splits(dsa.make_problem(C.DECODE_32K)) == 8      # 32 rows x 8 = 256
    assert dsa.attn_splits(dsa.make_problem(C.DECODE_128K)) == 16    # 8 rows x 16 = 128, capped by K / 128
    assert dsa.attn_splits(dsa.make_problem(C.PREFILL_8K)) == 1
    assert dsa.attn_splits(dsa.make_problem(C.PREFILL_64K_FP8)) == 1
    for batch in (1, 2, 3, 5, 8, 31, 64, 300):
        for topk in (1, 16, 100, 2048, 5000, 65536):
            p = _prob(dsa, C.DECODE_32K, batch=batch, topk=topk, kv_len=max(topk, 4096))
            s = dsa.attn_splits(p)
            assert s >= 1 and s & (s - 1) == 0 and s <= 32, (batch, topk, s)
            per = -(-topk // s)
            assert -(-per // 32) * 32 <= 2048, (batch, topk, s)       # one split's window fits in LDS
            if topk <= 4096:
                assert per >= min(128, topk), (batch, topk, s)               # at least 128 keys per split
            if batch * s > 256 and topk <= 65536 // 32:
                assert s == 1 or batch * s // 2 < 256, (batch, topk, s)     # no doubling past a full GPU
    assert dsa.attn_splits(_prob(dsa, C.DECODE_32K, q_len=0)) == 0


def _call_forward(dsa, p, ptr=16, ws_bytes=1 << 40, q_scale=None):
    L = dsa.lib()
    v = ctypes.c_void_p(ptr)
    return L.dsa_forward(ctypes.byref(p), v, q_scale, v, q_scale, v, v, v, None, v, None, v, ws_bytes, None)


def test_invalid_arguments_are_rejected_before_launch(dsa):
    L = dsa.lib()
    p = dsa.make_problem(C.DECODE_32K)
    # null pointers
    assert _call_forward(dsa, p, ptr=0) == dsa.DSA_ERR_INVALID_ARGUMENT
    # misaligned pointer
    assert _call_forward(dsa, p, ptr=24) == dsa.DSA_ERR_INVALID_ARGUMENT
    # workspace too small
    assert _call_forward(dsa, p, ws_bytes=16) == dsa.DSA_ERR_WORKSPACE_TOO_SMALL
    # bad dims
    for field, val in (("q_len", 0), ("kv_len", 0), ("topk", 0), ("batch", -1), ("v_dim", 1000)):
        bad = _prob(dsa, C.DECODE_32K, **{field: val})
        assert _call_forward(dsa, bad) == dsa.DSA_ERR_INVALID_ARGUMENT, field
    # q_len > kv_len
    assert _call_forward(dsa, _prob(dsa, C.DECODE_32K, q_len=40000)) == dsa.DSA_ERR_INVALID_ARGUMENT
    # non-finite scale
    assert _call_forward(dsa, _prob(dsa, C.DECODE_32K, softmax_scale=float("nan"))) == dsa.DSA_ERR_INVALID_ARGUMENT
    # unsupported: bf16 with non-V3.2 dims, mixed f32/bf16
    assert _call_forward(dsa, _prob(dsa, C.DECODE_32K, index_heads=32)) == dsa.DSA_ERR_UNSUPPORTED
    assert _call_forward(dsa, _prob(dsa, C.DECODE_32K, index_dtype=dsa.DSA_F32)) == dsa.DSA_ERR_UNSUPPORTED
    # latent gathers keep byte offsets below 2^31: (2^31 - 1) // 1152 rows
    assert (2 ** 31 - 1) // 1152 == 1864135
    assert _call_forward(dsa, _prob(dsa, C.DECODE_32K, kv_len=1864135 + 1)) == dsa.DSA_ERR_UNSUPPORTED
    assert dsa.workspace_size(_prob(dsa, C.DECODE_32K, batch=1, kv_len=1864135), dsa.DSA_OP_FORWARD) > 0
    assert _call_forward(dsa, _prob(dsa, C.DECODE_32K, topk=65537)) == dsa.DSA_ERR_UNSUPPORTED
    # fp8 without scales
    p8 = dsa.make_problem(C.PREFILL_64K_FP8)
    assert _call_forward(dsa, p8) == dsa.DSA_ERR_INVALID_ARGUMENT
    # top-k: row stride shorter than the row
    v = ctypes.c_void_p(16)
    assert L.dsa_topk(ctypes.byref(p), v, 100, v, None) == dsa.DSA_ERR_INVALID_ARGUMENT
    # attention: too small a workspace for the decode split
    need = dsa.workspace_size(p, dsa.DSA_OP_ATTN)
    assert need > 0
    assert L.dsa_sparse_mla_attn(ctypes.byref(p), v, v, v, v, None, v, need - 1, None) == \
        dsa.DSA_ERR_WORKSPACE_TOO_SMALL
    # timed forward: events requested but missing
    assert L.dsa_forward_timed(ctypes.byref(p), v, None, v, None, v, v, v, None, v, None, v, 1 << 40,
                               None, 8, None, None) == dsa.DSA_ERR_INVALID_ARGUMENT


def test_rotate_quantize_rejects_bad_arguments_without_launching(dsa):
    L = dsa.lib()
    v = ctypes.c_void_p(16)
    assert L.dsa_index_rotate_quantize(v, dsa.DSA_BF16, 0, 128, v, v, None) == dsa.DSA_OK      # nothing to do
    assert L.dsa_index_rotate_quantize(v, dsa.DSA_BF16, -1, 128, v, v, None) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert L.dsa_index_rotate_quantize(v, dsa.DSA_BF16, 8, 64, v, v, None) == dsa.DSA_ERR_UNSUPPORTED
    assert L.dsa_index_rotate_quantize(v, dsa.DSA_FP8_E4M3, 8, 128, v, v, None) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert L.dsa_index_rotate_quantize(None, dsa.DSA_BF16, 8, 128, v, v, None) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert L.dsa_index_rotate_quantize(ctypes.c_void_p(24), dsa.DSA_BF16, 8, 128, v, v, None) == \
        dsa.DSA_ERR_INVALID_ARGUMENT


def test_cache_append_checks_capacity_without_launching(dsa):
    L = dsa.lib()
    v = ctypes.c_void_p(16)
    p = dsa.make_problem(C.DECODE_32K, kv_capacity=32768)          # full: no room
    assert L.dsa_cache_append(ctypes.byref(p), 1, v, None, v, v, None, v, None) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert L.dsa_cache_append(ctypes.byref(p), 0, v, None, v, v, None, v, None) == dsa.DSA_OK
    p0 = dsa.make_problem(C.DECODE_32K)                            # capacity 0: nothing to append into
    assert L.dsa_cache_append(ctypes.byref(p0), 1, v, None, v, v, None, v, None) == dsa.DSA_ERR_INVALID_ARGUMENT
    small = dsa.make_problem(C.DECODE_32K, kv_capacity=100)        # capacity below kv_len
    assert _call_forward(dsa, small) == dsa.DSA_ERR_INVALID_ARGUMENT
    room = dsa.make_problem(C.DECODE_32K, kv_capacity=40000)
    assert L.dsa_cache_append(ctypes.byref(room), 4, v, None, None, v, None, v, None) == dsa.DSA_ERR_INVALID_ARGUMENT


def test_sliced_topk_plan_is_host_only_and_bounded(dsa):
    # few rows of 65536 positions or more get a workspace for the sliced
    # selection; many rows, shorter rows, and rows of at most K positions
    # select one work-group per row
    p4 = dsa.make_problem(C.DECODE_128K)
    need = dsa.workspace_size(p4, dsa.DSA_OP_TOPK)
    assert need >= 8 * 131072 * 12                    # kept lists and candidates can hold every position
    assert dsa.workspace_size(dsa.make_problem(C.DECODE_32K), dsa.DSA_OP_TOPK) == 0
    assert dsa.workspace_size(dsa.make_problem(C.PREFILL_8K), dsa.DSA_OP_TOPK) == 0
    assert dsa.workspace_size(_prob(dsa, C.DECODE_128K, batch=200), dsa.DSA_OP_TOPK) == 0
    assert dsa.workspace_size(_prob(dsa, C.DECODE_128K, kv_len=65535), dsa.DSA_OP_TOPK) == 0
    for batch, lk, k in ((1, 65536, 1), (8, 131072, 2048), (1, 1864135, 2048), (128, 70000, 4999), (3, 70001, 7)):
        n = dsa.workspace_size(_prob(dsa, C.DECODE_128K, batch=batch, kv_len=lk, topk=k), dsa.DSA_OP_TOPK)
        # row head + per-slice counts + row info + a (key, position) pair and a key per position
        assert n >= batch * ((4096 + 64) * 4 + 512 * 8 + 16 + lk * 12), (batch, lk, k)
        assert n <= batch * ((4096 + 64) * 4 + 512 * 8 + 16 + (lk + 4096) * 12), (batch, lk, k)
    # The forward's plan: decode rows of 16 or more 2048-key chunks select
    # from the indexer's candidate lists (256 slots per chunk up to 32
    # chunks, then as many as keep 8192 slots per row, when that leaves a
    # margin over a chunk's share s of the K chosen: s + 5 sqrt(s) + 16);
    # the sliced selection serves few long rows the lists do not.
    assert dsa.topk_list_slots(p4) == 128
    assert dsa.topk_list_slots(dsa.make_problem(C.DECODE_32K)) == 256
    assert dsa.topk_list_slots(_prob(dsa, C.DECODE_32K, kv_len=65536)) == 256
    assert dsa.topk_list_slots(_prob(dsa, C.DECODE_32K, kv_len=30720)) == 0      # 15 chunks
    assert dsa.topk_list_slots(_prob(dsa, C.DECODE_32K, kv_len=30721)) == 256    # 16 chunks
    assert dsa.topk_list_slots(_prob(dsa, C.DECODE_32K, topk=4097)) == 0        # share above 128
    assert dsa.topk_list_slots(_prob(dsa, C.DECODE_128K, kv_len=262144)) == 64   # 128 chunks
    assert dsa.topk_list_slots(_prob(dsa, C.DECODE_128K, kv_len=524288)) == 0    # 32 slots: no margin
    assert dsa.topk_list_slots(_prob(dsa, C.DECODE_128K, kv_len=1864135)) == 0   # 911 chunks of 8
    assert dsa.topk_list_slots(dsa.make_problem(C.PREFILL_8K)) == 0
    assert dsa.topk_list_slots(dsa.make_problem(C.TINY)) == 0
    assert dsa.topk_list_slots(_prob(dsa, C.DECODE_128K, q_len=0)) == 0
    # lists: 256 keys, 256 positions and a header per chunk
    assert dsa.workspace_size(p4, dsa.DSA_OP_FORWARD) >= 8 * 64 * (256 * 6 + 8)
    assert dsa.topk_slice_len(p4) == 0
    assert dsa.topk_slice_len(dsa.make_problem(C.DECODE_32K)) == 0
    big_k = _prob(dsa, C.DECODE_128K, topk=8192)
    assert dsa.topk_list_slots(big_k) == 0
    # 4096 positions per work-group for 8 rows of 128K (32 slices each)
    assert dsa.topk_slice_len(big_k) == 4096
    assert dsa.workspace_size(big_k, dsa.DSA_OP_FORWARD) >= dsa.workspace_size(big_k, dsa.DSA_OP_TOPK)
    assert dsa.topk_slice_len(_prob(dsa, C.DECODE_128K, batch=1, topk=8192)) == 1024
    assert dsa.topk_slice_len(_prob(dsa, C.DECODE_128K, q_len=0)) == 0


def test_static_forward_checks_before_any_hip_call(dsa):
    # fake but aligned device pointers: every rejection comes before the
    # scratch lookup or a launch, so this runs without a GPU
    L = dsa.lib()
    v = ctypes.c_void_p(256)
    big = dsa.make_problem(C.PREFILL_8K)
    assert dsa.workspace_size(big, dsa.DSA_OP_FORWARD) > dsa.DSA_STATIC_SCRATCH_BYTES
    args = [v] * 10 + [None]          # q_idx .. lse, stream
    assert L.dsa_forward_static(ctypes.byref(big), *args) == dsa.DSA_ERR_EXCEEDS_SCRATCH
    # both decode workloads fit, with or without top-k indices out
    for cfg in (C.DECODE_32K, C.DECODE_128K):
        assert dsa.workspace_size(dsa.make_problem(cfg), dsa.DSA_OP_FORWARD) <= dsa.DSA_STATIC_SCRATCH_BYTES
    p = dsa.make_problem(C.DECODE_32K)
    bad = list(args)
    bad[0] = None                      # no q_idx
    assert L.dsa_forward_static(ctypes.byref(p), *bad) == dsa.DSA_ERR_INVALID_ARGUMENT
    bad = list(args)
    bad[9] = ctypes.c_void_p(260)      # misaligned lse
    assert L.dsa_forward_static(ctypes.byref(p), *bad) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert L.dsa_forward_static(None, *args) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert "static scratch" in dsa.status_string(dsa.DSA_ERR_EXCEEDS_SCRATCH)
    assert dsa.DSA_STATIC_SCRATCH_BYTES == 96 << 20


def test_topk_ws_rejects_small_workspace_before_launch(dsa):
    L = dsa.lib()
    p = dsa.make_problem(C.DECODE_128K)
    v = ctypes.c_void_p(16)
    need = dsa.workspace_size(p, dsa.DSA_OP_TOPK)
    assert L.dsa_topk_ws(ctypes.byref(p), v, 131072, v, v, need - 1, None) == dsa.DSA_ERR_WORKSPACE_TOO_SMALL
    assert L.dsa_topk_ws(ctypes.byref(p), v, 131072, v, None, need, None) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert L.dsa_topk_ws(ctypes.byref(p), v, 100, v, v, need, None) == dsa.DSA_ERR_INVALID_ARGUMENT
