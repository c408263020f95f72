"""Throughput of the fused DSA hot path (indexer -> top-k -> sparse MLA) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]

A step is one dsa_forward call over one batch of synthetic inputs already
resident in HBM.  Input sets rotate between steps so that repeated steps do
not hit data left in the 256 MB Infinity Cache.  Prints one JSON line.
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


def source_hash(name):
    with open(os.path.join(ROOT, "sparse_attention_15_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel_src, workload):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if the
    kernel source is unchanged since they were taken; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("source_sha256_16") != source_hash(kernel_src):
        return None
    return rec.get("bytes_per_launch")


class _Same:
    """Indexable stand-in that returns one host array for any key."""

    def __init__(self, a):
        self.a = a

    def __getitem__(self, key):
        return self.a


def cpu_baseline(cfg, inp, budget_s=20.0):
    """The oracle (unchanged) on a bounded sample of the same workload."""
    import numpy as np
    import threadpoolctl
    from oracle import dsa_oracle as O

    def host(t):
        if t is None:
            return None
        return t.cpu().numpy() if t.dtype == __import__("torch").uint8 else t.float().cpu().numpy().astype(np.float64)

    rows = [(b, i) for b in range(cfg.batch) for i in range(cfg.q_len)]
    if cfg.q_len > 4:   # prefill: spread the sample over the causal range, latest rows first
        rows = rows[::-1][::max(1, len(rows) // 64)]
    info = threadpoolctl.threadpool_info()
    threads = max(p["num_threads"] for p in info) if info else 1
    seq = {}
    done = 0
    el = 0.0
    for (b, i) in rows:
        if b not in seq:          # host copy of this sequence's caches (not timed)
            seq = {b: {k: host(inp[k][b]) if inp[k] is not None else None for k in ("k_idx", "k_scale", "kv")}}
        q = {k: host(inp[k][b, i]) if inp[k] is not None else None for k in ("q_idx", "q_scale", "head_w", "q_attn")}
        wrap = lambda a: None if a is None else _Same(a)  # noqa: E731
        t0 = time.perf_counter()
        O.forward_rows(wrap(q["q_idx"]), wrap(q["q_scale"]), wrap(seq[b]["k_idx"]), wrap(seq[b]["k_scale"]),
                       wrap(q["head_w"]), wrap(q["q_attn"]), wrap(seq[b]["kv"]), [(b, i)],
                       cfg.q_len, cfg.topk, cfg.softmax_scale, cfg.v_dim)
        el += time.perf_counter() - t0
        done += 1
        if el > budget_s:
            break
    return dict(value=round(done / el, 3), unit="queries/s", cores=int(threads), kind="oracle",
                sample=f"{done} of {cfg.batch * cfg.q_len} queries of {cfg.name}, fp64 numpy oracle, "
                       f"{el:.1f} s of oracle time" + ("; rows spread over the causal range" if cfg.q_len > 4 else ""))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="decode_bf16_B32_ctx32768")
    ap.add_argument("--sets", type=int, default=3, help="rotating input sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--out-dtype", default=None)
    ap.add_argument("--plain-steps", type=int, default=0,
                    help="also time this many steps without per-kernel events (reported as ms_per_step_plain)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path, so --gpus must be 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_attention_15_amd as dsa
    from dsa_workloads import BY_NAME, generate

    cfg = BY_NAME[args.config]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    p = dsa.make_problem(cfg, out_dtype=args.out_dtype)
    nsets = max(1, args.sets if cfg.q_len <= 4 else min(args.sets, 2))
    sets = [generate(cfg, device=dev, set_index=s) for s in range(nsets)]
    ws = torch.empty(dsa.workspace_size(p, dsa.DSA_OP_FORWARD), dtype=torch.uint8, device=dev)
    odt = torch.float32 if p.out_dtype == dsa.DSA_F32 else torch.bfloat16
    outs = [torch.empty(cfg.batch, cfg.q_len, cfg.attn_heads, cfg.v_dim, dtype=odt, device=dev) for _ in sets]
    lses = [torch.empty(cfg.batch, cfg.q_len, cfg.attn_heads, dtype=torch.float32, device=dev) for _ in sets]
    n_chunks = dsa.forward_chunks(p)
    slots_per_step = n_chunks * dsa.DSA_NUM_STAGES

    def step(k, events=None, base=0):
        s = sets[k % nsets]
        ev = None
        if events is not None:
            import ctypes
            ev = ctypes.cast(ctypes.byref(events.arr, ctypes.sizeof(ctypes.c_void_p) * 2 * base),
                             ctypes.POINTER(ctypes.c_void_p))
        dsa.forward(p, s["q_idx"], s["q_scale"], s["k_idx"], s["k_scale"], s["head_w"], s["q_attn"], s["kv"],
                    out=outs[k % nsets], lse=lses[k % nsets], workspace=ws, events=ev,
                    n_events=2 * slots_per_step)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    # timed region, with per-kernel HIP events recorded on the launch stream
    events = dsa.StageEvents(args.steps * slots_per_step)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k, events, base=k * slots_per_step)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    plain_ms = None
    if args.plain_steps > 0:
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for k in range(args.plain_steps):
            step(k)
        torch.cuda.synchronize()
        plain_ms = (time.perf_counter() - t1) * 1e3 / args.plain_steps

    stage_ms = [0.0] * dsa.DSA_NUM_STAGES
    for k in range(args.steps):
        for c in range(n_chunks):
            for st in range(dsa.DSA_NUM_STAGES):
                stage_ms[st] += events.elapsed_ms(k * slots_per_step + c * dsa.DSA_NUM_STAGES + st)
    events.close()
    stage_ms = [x / args.steps for x in stage_ms]
    idx_launch_ms = stage_ms[0] / n_chunks     # average indexer launch duration

    al = algorithmic(cfg)
    ms_per_step = elapsed * 1e3 / args.steps
    qps = cfg.batch * cfg.q_len / (ms_per_step * 1e-3)
    decode = cfg.q_len <= 4
    if decode:
        idx_bytes_launch = al["index_bytes"] / n_chunks
        achieved = idx_bytes_launch / (idx_launch_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4),
                    traffic=measured_traffic("indexer.hip", cfg.name), kernel="idx_decode_kernel",
                    per_launch=f"{idx_bytes_launch} algorithmic bytes (index keys + q + head weights)")
    else:
        peak = MFMA_FP8_PEAK_TFLOPS if cfg.index_dtype == "fp8_e4m3" else MFMA_BF16_PEAK_TFLOPS
        fl_launch = al["index_flops"] / n_chunks
        achieved = fl_launch / (idx_launch_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=peak, unit="TFLOP/s",
                    frac=round(achieved / peak, 4), traffic=measured_traffic("indexer.hip", cfg.name),
                    kernel="idx_prefill_kernel", per_launch=f"{fl_launch} algorithmic flops (2*H*D per visible pair)")
    path_bytes = al["index_bytes"] + al["attn_bytes"]
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
        "config": {"workload": cfg.name, "batch": cfg.batch, "q_len": cfg.q_len, "kv_len": cfg.kv_len,
                   "index_heads": cfg.index_heads, "index_dim": cfg.index_dim, "topk": cfg.topk,
                   "attn_heads": cfg.attn_heads, "qk_dim": cfg.qk_dim, "v_dim": cfg.v_dim,
                   "query_chunks": n_chunks, "input_sets": nsets},
        "roofline": roof,
        "stage_ms": {name: round(v, 5) for name, v in zip(dsa.STAGE_NAMES, stage_ms)},
        "ms_per_step_plain": None if plain_ms is None else round(plain_ms, 5),
        "path_hbm_frac": round(path_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "path_algorithmic_bytes": path_bytes,
        "path_mfma_frac_bf16": round((al["index_flops"] + al["attn_flops"]) / (ms_per_step * 1e-3) / 1e12
                                     / MFMA_BF16_PEAK_TFLOPS, 4),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, sets[0])
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
