"""Host-side logic of bench.py (no GPU): the algorithmic work it prices
kernels against, the kernel it names per stage, the path-level targets, and
the argument checks that refuse runs it cannot measure."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from dsa_workloads import BY_NAME  # noqa: E402

C2 = BY_NAME["decode_bf16_B32_ctx32768"]
C3 = BY_NAME["prefill_bf16_L8192"]
C4 = BY_NAME["decode_bf16_B8_ctx131072"]


def test_decode_algorithmic_bytes_by_hand():
    al = bench.algorithmic(C2)
    # index keys (32 x 32768 rows of 128 bf16) + index queries (32 x 64 x 128
    # bf16) + head weights (32 x 64 fp32)
    assert al["index_bytes"] == 32 * 32768 * 256 + 32 * 64 * 128 * 2 + 32 * 64 * 4 == 268_967_936
    # 2048 gathered 1152-byte rows per query + q (128 x 576 bf16) + out
    # (128 x 512 bf16) + lse (128 fp32)
    assert al["attn_bytes"] == 32 * (2048 * 1152 + 128 * 1152 + 128 * 1024 + 128 * 4) == 84_426_752
    assert al["pairs"] == 32 * 32768 and al["selected"] == 32 * 2048


def test_prefill_algorithmic_flops_by_hand():
    al = bench.algorithmic(C3)
    pairs = 8192 * 8193 // 2                       # causal triangle including the diagonal
    assert al["pairs"] == pairs
    assert al["index_flops"] == 2 * 64 * 128 * pairs
    selected = sum(min(2048, i + 1) for i in range(8192))
    assert al["selected"] == selected
    assert al["attn_flops"] == 2 * 128 * (576 + 512) * selected


def test_stage_kernels_name_the_top_k_kernel():
    assert bench.stage_kernels(C2, 0)[1] == "topk_kernel"
    assert bench.stage_kernels(C2, 0, 256)[1] == "topk_cand_kernel"       # candidate lists
    assert bench.stage_kernels(C4, 0, 128)[1] == "topk_cand_kernel"
    for k in bench.stage_kernels(C2, 0, 256):
        assert k in bench.KERNELS
    assert bench.stage_kernels(C4, 4096)[1] == "tk_coop_kernel"            # 8 rows x 32 slices
    from dsa_workloads import scaled
    many = scaled(C4, batch=64)                                            # 2048 slices: three kernels
    assert bench.stage_kernels(many, 4096)[1].startswith("tk_hist_kernel")
    assert bench.stage_kernels(C3)[0] == "idx_prefill_kernel"
    for k in bench.stage_kernels(C4, 4096):
        assert k in bench.KERNELS


def test_decode_target_is_sixty_percent_of_hbm():
    al = bench.algorithmic(C2)
    path = al["index_bytes"] + al["attn_bytes"]
    t = bench.path_target(C2, al, path, 0.1, 0.046)
    goal_ms = path / (0.6 * 8e12) * 1e3
    assert t["goal_ms_per_step"] == pytest.approx(goal_ms, abs=1e-5)
    assert abs(goal_ms - 0.0736) < 5e-4
    assert not t["met"] and t["gap_ms_per_step"] == pytest.approx(0.1 - goal_ms, abs=1e-5)
    assert bench.path_target(C2, al, path, goal_ms * 0.99, 0.0)["met"]


def test_prefill_target_is_half_the_bf16_peak():
    al = bench.algorithmic(C3)
    ms_at_half = al["index_flops"] / (0.5 * 2.5e15) * 1e3
    assert bench.path_target(C3, al, 0, 4.0, ms_at_half * 0.99)["met"]
    assert not bench.path_target(C3, al, 0, 4.0, ms_at_half * 1.01)["met"]
    assert bench.path_target(BY_NAME["tiny_prefill_f32_L256"], al, 0, 1.0, 1.0) is None


def test_combine_bytes_follow_the_partial_precision():
    al = bench.algorithmic(C2)
    _, byts, unit, _, _ = bench.kernel_units(C2, "attn_combine_kernel", al, 1, 8)
    # 8 bf16 partials + fp32 LSEs read, bf16 out + fp32 lse written, per (query, head)
    assert unit == "GB/s" and byts == 32 * 128 * (8 * (512 * 2 + 4) + 512 * 2 + 4)


def _run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, env={**os.environ, "WORLD_SIZE": "1"})


def test_bench_refuses_more_than_one_gpu():
    r = _run_bench("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_bench_refuses_context_sweep_of_prefill_or_short_context():
    r = _run_bench("--config", "prefill_bf16_L8192", "--kv-len", "16384")
    assert r.returncode == 2 and "--kv-len" in r.stderr
    r = _run_bench("--kv-len", "1000")                     # below top-k 2048
    assert r.returncode == 2
