"""Throughput of the fused DSA hot path (indexer -> top-k -> sparse MLA) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]
    python bench.py --copy-calibration      (a 1 GiB copy, for scaling byte counters)

A step is one dsa_forward call over one batch of synthetic inputs already
resident in HBM.  Input sets rotate between steps so that repeated steps do
not hit data left in the 256 MB Infinity Cache.  The timed region is `steps`
plain calls; per-kernel durations come from the same number of calls again
with a HIP event pair around every launch.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense, published
MFMA_FP8_PEAK_TFLOPS = 5000.0


def algorithmic(cfg):
    """Algorithmic bytes / flops of one call (what the method must move or compute)."""
    B, Lq, Lk, H, D, K = cfg.batch, cfg.q_len, cfg.kv_len, cfg.index_heads, cfg.index_dim, cfg.topk
    NH, Dqk, Dv = cfg.attn_heads, cfg.qk_dim, cfg.v_dim
    ib = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[cfg.index_dtype]
    ab = {"f32": 4, "bf16": 2}[cfg.attn_dtype]
    pairs = sum(Lk - Lq + i + 1 for i in range(Lq)) * B                  # visible (query, key) pairs
    sel = sum(min(K, Lk - Lq + i + 1) for i in range(Lq)) * B             # selected (query, key) pairs
    scale_b = (B * Lq * H + B * Lk) if cfg.index_dtype == "fp8_e4m3" else 0
    idx_bytes = B * Lk * D * ib + B * Lq * H * D * ib + B * Lq * H * 4 + scale_b
    # decode-shaped: every selected row is a distinct HBM read; prefill: the cache is read once
    gathered = sel * Dqk * ab if Lq <= 4 else B * Lk * Dqk * ab
    attn_bytes = gathered + B * Lq * NH * Dqk * ab + B * Lq * NH * Dv * ab + B * Lq * NH * 4
    return dict(pairs=pairs, selected=sel, index_bytes=idx_bytes, attn_bytes=attn_bytes,
                index_flops=2 * H * D * pairs, attn_flops=2 * NH * (Dqk + Dv) * sel)


# kernel -> (source file, stage index)
KERNELS = {
    "idx_decode_kernel": ("indexer.hip", 0),
    "idx_prefill_kernel": ("indexer.hip", 0),
    "idx_f32_kernel": ("indexer.hip", 0),
    "topk_kernel": ("topk.hip", 1),
    "topk_cand_kernel": ("topk.hip", 1),
    "tk_coop_kernel": ("topk_sliced.hip", 1),
    "tk_hist_kernel + tk_classify_kernel + tk_emit_kernel": ("topk_sliced.hip", 1),
    "attn_bf16_kernel": ("sparse_mla.hip", 2),
    "attn_f32_kernel": ("sparse_mla.hip", 2),
    "attn_combine_kernel": ("sparse_mla.hip", 3),
}


def source_hash(name):
    with open(os.path.join(ROOT, "sparse_attention_15_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), if
    the kernel's source is unchanged since the counters were taken; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}.{workload}.traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(KERNELS[kernel][0]):
        return None
    return rec.get("bytes_per_launch")


def stage_kernels(cfg, slice_len=0, list_slots=0):
    """Kernel that runs in each stage of dsa_forward for this workload.

    list_slots > 0: the top-k selects from the indexer's per-chunk candidate
    lists (one work-group per row).  slice_len > 0: the top-k cuts each row
    into slices of that many positions, one work-group each; all slices of
    the launch run together in one cooperative kernel when they fit on the
    chip at once (256 CUs hold at least one work-group each), else in three
    kernels."""
    decode = cfg.q_len <= 4
    topk = "topk_kernel"
    if list_slots > 0:
        topk = "topk_cand_kernel"
    elif slice_len > 0:
        slices = cfg.batch * cfg.q_len * -(-cfg.kv_len // slice_len)
        topk = "tk_coop_kernel" if slices <= 256 else "tk_hist_kernel + tk_classify_kernel + tk_emit_kernel"
    if cfg.index_dtype == "f32":
        return ["idx_f32_kernel", topk, "attn_f32_kernel", "attn_combine_kernel"]
    return ["idx_decode_kernel" if decode else "idx_prefill_kernel", topk, "attn_bf16_kernel",
            "attn_combine_kernel"]


def kernel_units(cfg, kernel, al, n_chunks, split_rows):
    """(bound, algorithmic units per launch, unit, peak, description) of one kernel."""
    B, Lq, Lk, K = cfg.batch, cfg.q_len, cfg.kv_len, cfg.topk
    NH, Dv = cfg.attn_heads, cfg.v_dim
    decode = Lq <= 4
    if kernel.startswith("idx_"):
        if decode or cfg.index_dtype == "f32":
            return ("hbm", al["index_bytes"] / n_chunks, "GB/s", HBM_PEAK_GBS,
                    "algorithmic bytes per launch: index keys + index q + head weights (+ scales)")
        peak = MFMA_FP8_PEAK_TFLOPS if cfg.index_dtype == "fp8_e4m3" else MFMA_BF16_PEAK_TFLOPS
        return ("mfma", al["index_flops"] / n_chunks, "TFLOP/s", peak,
                "algorithmic flops per launch: 2*H*D per visible (query, key) pair")
    if kernel.startswith("topk_") or kernel.startswith("tk_"):
        return ("hbm", 4 * al["pairs"] / n_chunks, "GB/s", HBM_PEAK_GBS,
                "algorithmic bytes per launch: one fp32 score per visible (query, key) pair")
    if kernel.startswith("attn_") and kernel != "attn_combine_kernel":
        if decode:
            return ("hbm", al["attn_bytes"] / n_chunks, "GB/s", HBM_PEAK_GBS,
                    "algorithmic bytes per launch: selected latent rows + q + out + lse")
        return ("mfma", al["attn_flops"] / n_chunks, "TFLOP/s", MFMA_BF16_PEAK_TFLOPS,
                "algorithmic flops per launch: 2*NH*(Dqk+Dv) per selected (query, key) pair")
    # combine: read the partials (output precision) and LSEs of every split,
    # write out and lse
    ob = 4 if cfg.index_dtype == "f32" else 2
    rows = B * Lq / n_chunks
    byts = rows * NH * (split_rows * (Dv * ob + 4) + Dv * ob + 4)
    return ("hbm", byts, "GB/s", HBM_PEAK_GBS,
            "bytes per launch: split partials (output precision) and LSEs read + out and lse written")


DECODE_HBM_TARGET = 0.60        # decode-shaped path: fraction of HBM bandwidth
PREFILL_INDEX_TARGET = 0.50     # prefill-shaped indexer: fraction of the bf16 MFMA peak


def path_target(cfg, al, path_bytes, ms_per_step, index_ms):
    """The step against the path-level targets: decode-shaped workloads move
    the path's algorithmic bytes at >= 60% of HBM; prefill-shaped ones run
    the indexer at >= 50% of the bf16 MFMA peak (index_ms: the indexer's
    event time per step)."""
    if cfg.q_len <= 4:
        frac = path_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS
        need_ms = path_bytes / (DECODE_HBM_TARGET * HBM_PEAK_GBS * 1e9) * 1e3
        return {"what": "decode path algorithmic bytes at >= 60% of 8 TB/s", "value": round(frac, 4),
                "goal": DECODE_HBM_TARGET, "met": frac >= DECODE_HBM_TARGET,
                "goal_ms_per_step": round(need_ms, 5), "gap_ms_per_step": round(max(0.0, ms_per_step - need_ms), 5)}
    if cfg.index_dtype == "f32":
        return None
    frac = al["index_flops"] / (index_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS
    return {"what": "prefill indexer flops at >= 50% of the 2.5 PFLOP/s bf16 peak (indexer event time)",
            "value": round(frac, 4), "goal": PREFILL_INDEX_TARGET, "met": frac >= PREFILL_INDEX_TARGET}


class _Same:
    """Indexable stand-in that returns one host array for any key."""

    def __init__(self, a):
        self.a = a

    def __getitem__(self, key):
        return self.a


def cpu_baseline(cfg, sets, budget_s=12.0):
    """The oracle (unchanged) on a bounded sample of the same workload: query
    rows in a fixed order, cycling over the input sets, until about budget_s
    seconds of oracle time (at least one row)."""
    import numpy as np
    import threadpoolctl
    import torch
    from oracle import dsa_oracle as O

    def host(t):
        if t is None:
            return None
        return t.cpu().numpy() if t.dtype == torch.uint8 else t.float().cpu().numpy().astype(np.float64)

    rows = [(b, i) for b in range(cfg.batch) for i in range(cfg.q_len)]
    if cfg.q_len > 4:   # prefill: spread the sample over the causal range, latest rows first
        rows = rows[::-1][::max(1, len(rows) // 64)]
    info = threadpoolctl.threadpool_info()
    threads = max(p["num_threads"] for p in info) if info else 1
    cache_key, seq = None, None
    done, el = 0, 0.0
    passes = 0
    while el <= budget_s:
        for si, inp in enumerate(sets):
            for (b, i) in rows:
                if cache_key != (si, b):          # host copy of this sequence's caches (not timed)
                    seq = {k: host(inp[k][b]) if inp[k] is not None else None for k in ("k_idx", "k_scale", "kv")}
                    cache_key = (si, b)
                q = {k: host(inp[k][b, i]) if inp[k] is not None else None
                     for k in ("q_idx", "q_scale", "head_w", "q_attn")}
                wrap = lambda a: None if a is None else _Same(a)  # noqa: E731
                t0 = time.perf_counter()
                O.forward_rows(wrap(q["q_idx"]), wrap(q["q_scale"]), wrap(seq["k_idx"]), wrap(seq["k_scale"]),
                               wrap(q["head_w"]), wrap(q["q_attn"]), wrap(seq["kv"]), [(b, i)],
                               cfg.q_len, cfg.topk, cfg.softmax_scale, cfg.v_dim)
                el += time.perf_counter() - t0
                done += 1
                if el > budget_s:
                    break
            if el > budget_s:
                break
        passes += 1
    return dict(value=round(done / el, 3), unit="queries/s", cores=int(threads), kind="oracle",
                sample=f"{done} query rows of {cfg.name} ({len(rows)} distinct rows per input set"
                       + (", spread over the causal range" if cfg.q_len > 4 else "")
                       + f", {len(sets)} input sets cycled), fp64 numpy oracle, {el:.1f} s of oracle time")


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain elementwise copy of known size (nbytes read, nbytes written)
    for scaling the FETCH_SIZE / WRITE_SIZE counters of a rocprofv3 run."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps,
                      "copy_GBps_read_plus_write": round(2 * nbytes / el / 1e9, 1)}), flush=True)


def graph_call_ms(fn, torch, reps=20):
    """Average duration of one fn() call: `reps` calls captured in a HIP graph
    and replayed, so host submission time does not enter the measurement."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (3 * reps)


def decode_loop(args, cfg, dsa, generate, torch):
    """Multi-step decode with cache appends: contexts L0+1 .. Lk, one query per
    sequence per step."""
    from dsa_workloads import scaled
    if cfg.q_len != 1:
        print("--decode-loop applies to decode workloads (one query per sequence)", file=sys.stderr)
        sys.exit(2)
    N = args.steps
    L0 = cfg.kv_len - N
    # the full caches at the final context, and N queries: step t is row t of
    # the causal problem with Lq = N, Lk = L0 + N
    full = generate(scaled(cfg, q_len=N), device="cuda:0")
    B, cap = cfg.batch, cfg.kv_len
    k_c = full["k_idx"].clone()
    ks_c = full["k_scale"].clone() if full["k_scale"] is not None else None
    kv_c = full["kv"].clone()
    new_k = [full["k_idx"][:, L0 + t:L0 + t + 1].contiguous() for t in range(N)]
    new_ks = [full["k_scale"][:, L0 + t:L0 + t + 1].contiguous() if ks_c is not None else None for t in range(N)]
    new_kv = [full["kv"][:, L0 + t:L0 + t + 1].contiguous() for t in range(N)]
    qs = {k: [full[k][:, t:t + 1].contiguous() if full[k] is not None else None for t in range(N)]
          for k in ("q_idx", "q_scale", "head_w", "q_attn")}
    probs_app = [dsa.make_problem(scaled(cfg, kv_len=L0 + t), kv_capacity=cap) for t in range(N)]
    probs_fwd = [dsa.make_problem(scaled(cfg, kv_len=L0 + t + 1), kv_capacity=cap) for t in range(N)]
    ws = torch.empty(max(dsa.workspace_size(pp, dsa.DSA_OP_FORWARD) for pp in probs_fwd), dtype=torch.uint8,
                     device="cuda:0")
    odt = torch.float32 if probs_fwd[0].out_dtype == dsa.DSA_F32 else torch.bfloat16
    out = torch.empty(B, 1, cfg.attn_heads, cfg.v_dim, dtype=odt, device="cuda:0")
    lse = torch.empty(B, 1, cfg.attn_heads, dtype=torch.float32, device="cuda:0")
    ev = []

    def run(record):
        for t in range(N):
            if record:
                e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                e[0].record()
            dsa.cache_append(probs_app[t], new_k[t], new_ks[t], new_kv[t], k_c, ks_c, kv_c)
            if record:
                e[1].record()
            dsa.forward(probs_fwd[t], qs["q_idx"][t], qs["q_scale"][t], k_c, ks_c, qs["head_w"][t],
                        qs["q_attn"][t], kv_c, out=out, lse=lse, workspace=ws)
            if record:
                e[2].record()
                ev.append(e)

    for _ in range(max(1, args.warmup // max(1, N))):
        run(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(False)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    run(True)
    torch.cuda.synchronize()
    app = [e[0].elapsed_time(e[1]) for e in ev]
    fwd = [e[1].elapsed_time(e[2]) for e in ev]
    t_last = N - 1
    app_graph_ms = graph_call_ms(lambda: dsa.cache_append(probs_app[t_last], new_k[t_last], new_ks[t_last],
                                                          new_kv[t_last], k_c, ks_c, kv_c), torch)
    ms = el * 1e3 / N
    res = {
        "metric": "DSA queries/sec (indexer+top-k+sparse MLA)",
        "value": round(B * N / el, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": N,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f32": "f32", "fp8_e4m3": "fp8_e4m3+bf16"}[cfg.index_dtype],
        "data": "synthetic (seeded generators; no dataset or weights)",
        "config": {"workload": cfg.name + "+decode_loop", "batch": B, "q_len": 1,
                   "start_context": L0 + 1, "end_context": L0 + N, "kv_capacity": cap,
                   "index_heads": cfg.index_heads, "index_dim": cfg.index_dim, "topk": cfg.topk,
                   "attn_heads": cfg.attn_heads, "qk_dim": cfg.qk_dim, "v_dim": cfg.v_dim},
        "decode_loop": {"append_us": round(1e3 * app_graph_ms, 2), "append_us_in_step": round(1e3 * sum(app) / N, 2),
                        "forward_ms_first": round(fwd[0], 5), "forward_ms_last": round(fwd[-1], 5),
                        "forward_ms_mean": round(sum(fwd) / N, 5),
                        "note": "each step: append one token per sequence (index key + latent row), then "
                                "one query per sequence at the grown context; events bracket each call "
                                "(append_us: one append from 20 replayed as a HIP graph)"},
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="decode_bf16_B32_ctx32768")
    ap.add_argument("--sets", type=int, default=3, help="rotating input sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--out-dtype", default=None)
    ap.add_argument("--with-producer", action="store_true",
                    help="FP8-index workloads: start each step from bf16 index activations and run the FP8 "
                         "producer (Hadamard rotation + ue8m0/E4M3 quantisation) before the fused path")
    ap.add_argument("--with-projections", action="store_true",
                    help="bf16-index workloads: each step first projects the index queries from a query latent "
                         "and the head weights from a hidden state, and un-absorbs the attention output after "
                         "(bf16 GEMMs on synthetic weights)")
    ap.add_argument("--decode-loop", action="store_true",
                    help="decode workloads: each step appends one token per sequence to caches with room for "
                         "them and runs the fused path for one query at the grown context; the `steps` "
                         "steps end at the workload's context")
    ap.add_argument("--kv-len", type=int, default=None,
                    help="decode workloads: run the workload at this context instead (same batch, top-k and "
                         "planted fraction; the workload name gets ctx<kv-len>), for context sweeps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB elementwise copy (for calibrating rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path, so --gpus must be 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return
    import torch
    import sparse_attention_15_amd as dsa
    from dsa_workloads import BY_NAME, generate

    cfg = BY_NAME[args.config]
    if args.kv_len is not None:
        if cfg.q_len > 4 or args.kv_len < cfg.topk or "_ctx" not in cfg.name:
            print("--kv-len applies to decode workloads, at a context of at least top-k", file=sys.stderr)
            sys.exit(2)
        from dsa_workloads import scaled
        plants = cfg.plant_count
        if cfg.planting == "fraction":            # keep the planted fraction of the context
            plants = max(1, round(cfg.plant_count * args.kv_len / cfg.kv_len))
        cfg = scaled(cfg, kv_len=args.kv_len, plant_count=plants,
                     name=cfg.name[:cfg.name.index("_ctx")] + f"_ctx{args.kv_len}")
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.decode_loop:
        decode_loop(args, cfg, dsa, generate, torch)
        return
    p = dsa.make_problem(cfg, out_dtype=args.out_dtype)
    nsets = max(1, args.sets if cfg.q_len <= 4 else min(args.sets, 2))
    producer = args.with_producer
    if producer and cfg.index_dtype != "fp8_e4m3":
        print("--with-producer applies to FP8-index workloads only", file=sys.stderr)
        sys.exit(2)
    if producer:
        # bf16 index activations of the same shapes; the FP8 inputs are
        # produced inside every step
        from dsa_workloads import scaled
        cfg16 = scaled(cfg, index_dtype="bf16")
        sets = [generate(cfg16, device=dev, set_index=s) for s in range(nsets)]
        for st_ in sets:
            st_["q_codes"] = torch.empty(st_["q_idx"].shape, dtype=torch.uint8, device=dev)
            st_["q_scale"] = torch.empty(st_["q_idx"].shape[:-1], dtype=torch.uint8, device=dev)
            st_["k_codes"] = torch.empty(st_["k_idx"].shape, dtype=torch.uint8, device=dev)
            st_["k_scale"] = torch.empty(st_["k_idx"].shape[:-1], dtype=torch.uint8, device=dev)
    else:
        sets = [generate(cfg, device=dev, set_index=s) for s in range(nsets)]
    projections = args.with_projections
    if projections:
        if cfg.index_dtype != "bf16" or producer or p.out_dtype != dsa.DSA_BF16:
            print("--with-projections applies to bf16-index workloads with bf16 output", file=sys.stderr)
            sys.exit(2)
        from dsa_workloads import generate_projection_inputs
        from dsa_workloads.generate import V_HEAD_DIM
        for si, st_ in enumerate(sets):
            st_.update(generate_projection_inputs(cfg, device=dev, set_index=si))
            st_["q_proj"] = torch.empty_like(st_["q_idx"])
            st_["w_out"] = torch.empty_like(st_["head_w"])
            st_["o_final"] = torch.empty(cfg.batch, cfg.q_len, cfg.attn_heads, V_HEAD_DIM, dtype=torch.bfloat16,
                                         device=dev)
            nws = dsa.head_weights_workspace_size(p, st_["x"].shape[-1])
            st_["w_ws"] = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
    proj_ev = []
    ws = torch.empty(dsa.workspace_size(p, dsa.DSA_OP_FORWARD), dtype=torch.uint8, device=dev)
    odt = torch.float32 if p.out_dtype == dsa.DSA_F32 else torch.bfloat16
    outs = [torch.empty(cfg.batch, cfg.q_len, cfg.attn_heads, cfg.v_dim, dtype=odt, device=dev) for _ in sets]
    lses = [torch.empty(cfg.batch, cfg.q_len, cfg.attn_heads, dtype=torch.float32, device=dev) for _ in sets]
    n_chunks = dsa.forward_chunks(p)
    slots_per_step = n_chunks * dsa.DSA_NUM_STAGES

    prod_ev = []

    def step(k, events=None, base=0):
        s = sets[k % nsets]
        q_idx, k_idx = s["q_idx"], s["k_idx"]
        if producer:
            if events is not None:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
            dsa.index_rotate_quantize(s["q_idx"], s["q_codes"], s["q_scale"])
            dsa.index_rotate_quantize(s["k_idx"], s["k_codes"], s["k_scale"])
            if events is not None:
                e1.record()
                prod_ev.append((e0, e1))
            q_idx, k_idx = s["q_codes"], s["k_codes"]
        head_w = s["head_w"]
        if projections:
            if events is not None:
                pe = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
                pe[0].record()
            dsa.index_q_proj(p, s["cq"], s["wq_b"], out=s["q_proj"])
            if events is not None:
                pe[1].record()
            dsa.head_weights_proj(p, s["x"], s["w_proj"], out=s["w_out"], workspace=s["w_ws"])
            if events is not None:
                pe[2].record()
            q_idx, head_w = s["q_proj"], s["w_out"]
        ev = None
        if events is not None:
            import ctypes
            ev = ctypes.cast(ctypes.byref(events.arr, ctypes.sizeof(ctypes.c_void_p) * 2 * base),
                             ctypes.POINTER(ctypes.c_void_p))
        dsa.forward(p, q_idx, s["q_scale"], k_idx, s["k_scale"], head_w, s["q_attn"], s["kv"],
                    out=outs[k % nsets], lse=lses[k % nsets], workspace=ws, events=ev,
                    n_events=2 * slots_per_step)
        if projections:
            if events is not None:
                pe[3].record()
            dsa.out_unabsorb(p, outs[k % nsets], s["w_uv"], out=s["o_final"])
            if events is not None:
                pe[4].record()
                proj_ev.append(pe)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    # timed region: exactly `steps` calls, no instrumentation
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # per-kernel durations: the same calls again with a HIP event pair around
    # every launch, recorded on the stream the kernels run on
    ksteps = args.steps
    events = dsa.StageEvents(ksteps * slots_per_step)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for k in range(ksteps):
        step(k, events, base=k * slots_per_step)
    torch.cuda.synchronize()
    evented_ms = (time.perf_counter() - t1) * 1e3 / ksteps
    stage_ms = [0.0] * dsa.DSA_NUM_STAGES
    for k in range(ksteps):
        for c in range(n_chunks):
            for st in range(dsa.DSA_NUM_STAGES):
                stage_ms[st] += events.elapsed_ms(k * slots_per_step + c * dsa.DSA_NUM_STAGES + st)
    events.close()
    stage_ms = [x / ksteps for x in stage_ms]

    al = algorithmic(cfg)
    ms_per_step = elapsed * 1e3 / args.steps
    qps = cfg.batch * cfg.q_len / (ms_per_step * 1e-3)
    kernels = stage_kernels(cfg, dsa.topk_slice_len(p), dsa.topk_list_slots(p))
    splits = dsa.attn_splits(p)
    dom = max(range(dsa.DSA_NUM_STAGES), key=lambda st: stage_ms[st])
    kname = kernels[dom]
    launch_ms = stage_ms[dom] / n_chunks               # average launch duration of that kernel
    bound, units, unit, peak, desc = kernel_units(cfg, kname, al, n_chunks, splits)
    scale = 1e9 if unit == "GB/s" else 1e12
    achieved = units / (launch_ms * 1e-3) / scale
    roof = dict(bound=bound, achieved=round(achieved, 1), peak=peak, unit=unit, frac=round(achieved / peak, 4),
                traffic=measured_traffic(kname, cfg.name), kernel=kname,
                launch_us=round(launch_ms * 1e3, 2), per_launch=f"{units:.0f} {desc}")
    path_bytes = al["index_bytes"] + al["attn_bytes"]
    prod = None
    if producer:
        prod_ms = sum(a.elapsed_time(b) for a, b in prod_ev) / max(1, len(prod_ev))
        prows = cfg.batch * cfg.q_len * cfg.index_heads + cfg.batch * cfg.kv_len
        pbytes = prows * (cfg.index_dim * 2 + cfg.index_dim + 1)      # bf16 in, codes + scale byte out
        gbs = pbytes / (prod_ms * 1e-3) / 1e9
        prod = dict(kernel="rotate_quant_kernel", rows_per_step=prows, ms_per_step=round(prod_ms, 5),
                    algorithmic_bytes=pbytes, achieved=round(gbs, 1), unit="GB/s", peak=HBM_PEAK_GBS,
                    frac=round(gbs / HBM_PEAK_GBS, 4),
                    note="q rows (B*Lq*H) and key rows (B*Lk): 128 bf16 in, 128 E4M3 codes + 1 scale byte out")
    proj = None
    if projections:
        M = cfg.batch * cfg.q_len
        s0 = sets[0]
        R, hid = s0["cq"].shape[-1], s0["x"].shape[-1]
        HD, H, NH, Dv, V = cfg.index_heads * cfg.index_dim, cfg.index_heads, cfg.attn_heads, cfg.v_dim, V_HEAD_DIM
        work = {  # (algorithmic bytes, flops) per call: operands read once, output written once
            "index_q": (2 * (M * R + HD * R + M * HD), 2 * M * HD * R),
            "head_weights": (2 * (M * hid + H * hid) + 4 * M * H, 2 * M * H * hid),
            "unabsorb": (2 * (M * NH * Dv + NH * V * Dv + M * NH * V), 2 * M * NH * V * Dv),
        }
        calls = {
            "index_q": lambda: dsa.index_q_proj(p, s0["cq"], s0["wq_b"], out=s0["q_proj"]),
            "head_weights": lambda: dsa.head_weights_proj(p, s0["x"], s0["w_proj"], out=s0["w_out"],
                                                          workspace=s0["w_ws"]),
            "unabsorb": lambda: dsa.out_unabsorb(p, outs[0], s0["w_uv"], out=s0["o_final"]),
        }
        slots = {"index_q": (0, 1), "head_weights": (1, 2), "unabsorb": (3, 4)}
        kern = "gemm_skinny_kernel" if M <= 32 else "gemm_tile_kernel / gemm_big_kernel"
        # each GEMM against the roof its arithmetic intensity puts it under
        ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        proj = {"kernel": kern}
        for name, (a_, b_) in slots.items():
            in_step = sum(e[a_].elapsed_time(e[b_]) for e in proj_ev) / max(1, len(proj_ev))
            ms_ = graph_call_ms(calls[name], torch)
            nbytes, flops = work[name]
            if flops / nbytes < ridge:
                ach = nbytes / (ms_ * 1e-3) / 1e9
                proj[name] = dict(bound="hbm", ms=round(ms_, 5), ms_in_step=round(in_step, 5),
                                  algorithmic_bytes=nbytes, achieved=round(ach, 1), unit="GB/s", peak=HBM_PEAK_GBS,
                                  frac=round(ach / HBM_PEAK_GBS, 4))
            else:
                ach = flops / (ms_ * 1e-3) / 1e12
                proj[name] = dict(bound="mfma", ms=round(ms_, 5), ms_in_step=round(in_step, 5), flops=flops,
                                  achieved=round(ach, 1), unit="TFLOP/s", peak=MFMA_BF16_PEAK_TFLOPS,
                                  frac=round(ach / MFMA_BF16_PEAK_TFLOPS, 4))
        proj["note"] = ("inside every step: index queries from a [T,%d] latent, head weights from a [T,%d] hidden "
                        "state, per-head un-absorption to v_head_dim %d.  ms: one call, from 20 calls replayed as a "
                        "HIP graph; ms_in_step: events around the call inside the timed steps (includes host "
                        "submission gaps for short kernels)" % (R, hid, V))
    res = {
        "metric": "DSA queries/sec (indexer+top-k+sparse MLA)",
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f32": "f32", "fp8_e4m3": "fp8_e4m3+bf16"}[cfg.index_dtype],
        "data": "synthetic (seeded generators; no dataset or weights)",
        "config": {"workload": cfg.name + ("+fp8_producer" if producer else "") + ("+projections" if projections else ""), "batch": cfg.batch, "q_len": cfg.q_len, "kv_len": cfg.kv_len,
                   "index_heads": cfg.index_heads, "index_dim": cfg.index_dim, "topk": cfg.topk,
                   "attn_heads": cfg.attn_heads, "qk_dim": cfg.qk_dim, "v_dim": cfg.v_dim,
                   "query_chunks": n_chunks, "attn_splits": splits, "input_sets": nsets},
        "roofline": roof,
        "stage_ms": {name: round(v, 5) for name, v in zip(dsa.STAGE_NAMES, stage_ms)},
        "ms_per_step_evented": round(evented_ms, 5),
        **({"producer": prod} if prod else {}),
        **({"projections": proj} if proj else {}),
        "path_hbm_frac": round(path_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "path_algorithmic_bytes": path_bytes,
        "path_mfma_frac_bf16": round((al["index_flops"] + al["attn_flops"]) / (ms_per_step * 1e-3) / 1e12
                                     / MFMA_BF16_PEAK_TFLOPS, 4),
        "target": path_target(cfg, al, path_bytes, ms_per_step, stage_ms[0]),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, sets)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
