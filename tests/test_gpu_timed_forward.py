"""dsa_forward_timed: the forward with a HIP event pair per (chunk, stage).

The events ride on the stage's own launches (the first kernel's start, the
last kernel's end), or are recorded by themselves when a stage launches
nothing (the combine of an unsplit launch).  The timed call must give the
plain call's results bit for bit, leave every event pair recorded with a
non-negative elapsed time, and leave no timing attached to later calls.
"""
import math

import pytest
import torch

import sparse_attention_15_amd as dsa
from dsa_workloads import configs as C
from dsa_workloads import generate

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAMES = ("q_idx", "q_scale", "k_idx", "k_scale", "head_w", "q_attn", "kv")

CASES = [
    # decode: candidate-list top-k, 8 splits and the combine launch
    C.scaled(C.DECODE_32K, name="timed_decode_b2_L32768", batch=2, kv_len=32768, plant_count=300),
    # decode, few long rows: the sliced top-k (several launches in one stage)
    C.scaled(C.DECODE_128K, name="timed_decode_b2_L70000", batch=2, kv_len=70000, topk=8192, plant_count=100),
    # prefill: one work-group per query, no split, so the combine stage launches nothing
    C.scaled(C.PREFILL_8K, name="timed_prefill_L1500", q_len=1500, kv_len=1500),
    # FP8 prefill large enough to run in several query chunks
    C.scaled(C.PREFILL_64K_FP8, name="timed_fp8_L20000", q_len=20000, kv_len=20000),
]


def _run(p, inp, events=None, n_events=0):
    idx = torch.empty(p.batch, p.q_len, p.topk, dtype=torch.int32, device=DEV)
    lse = torch.empty(p.batch, p.q_len, p.attn_heads, dtype=torch.float32, device=DEV)
    out, lse, idx = dsa.forward(p, *[inp[n] for n in NAMES], lse=lse, topk_idx=idx, events=events,
                                n_events=n_events)
    return out, lse, idx


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_timed_forward_equals_plain_and_records_every_stage(cfg):
    inp = generate(cfg, device=DEV)
    p = dsa.make_problem(cfg)
    ref = _run(p, inp)
    torch.cuda.synchronize()
    n_slots = dsa.forward_chunks(p) * dsa.DSA_NUM_STAGES
    ev = dsa.StageEvents(n_slots)
    try:
        got = _run(p, inp, ev.arr, ev.n)
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert torch.equal(a, b), cfg.name
        for slot in range(n_slots):
            ms = ev.elapsed_ms(slot)
            assert math.isfinite(ms) and ms >= 0.0, (cfg.name, slot, ms)
    finally:
        torch.cuda.synchronize()
        ev.close()
    # the events are gone: later untimed calls must not refer to them
    again = _run(p, inp)
    scores = dsa.index_scores(p, inp["q_idx"], inp["q_scale"], inp["k_idx"], inp["k_scale"], inp["head_w"])
    torch.cuda.synchronize()
    for a, b in zip(ref, again):
        assert torch.equal(a, b), cfg.name
    assert scores.shape[-1] == cfg.kv_len


def test_timed_forward_with_fewer_slots_than_stages():
    # only the first chunk's stages are timed; the rest of the call runs untimed
    cfg = C.scaled(C.PREFILL_64K_FP8, name="timed_fp8_partial", q_len=20000, kv_len=20000)
    inp = generate(cfg, device=DEV)
    p = dsa.make_problem(cfg)
    assert dsa.forward_chunks(p) > 1
    ref = _run(p, inp)
    ev = dsa.StageEvents(dsa.DSA_NUM_STAGES)
    try:
        got = _run(p, inp, ev.arr, ev.n)
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
        for slot in range(dsa.DSA_NUM_STAGES):
            assert ev.elapsed_ms(slot) >= 0.0
    finally:
        torch.cuda.synchronize()
        ev.close()
