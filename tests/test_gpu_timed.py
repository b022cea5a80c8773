"""ttt_la_forward_timed: the same results as ttt_la_forward, bit for bit, and
events that bracket a kernel of positive duration, in every mode."""
import numpy as np
import pytest
import torch

from helpers import la, to_device, workloads

CASES = [
    workloads.make_spec("per_token_linear", 1, 2, 300, 128, chunk=64, dtype="bf16"),
    workloads.make_spec("per_token_linear", 1, 2, 300, 64, chunk=32, dtype="fp32"),
    workloads.make_spec("large_chunk_linear", 1, 2, 1000, 64, chunk=256, dtype="bf16"),
    workloads.make_spec("large_chunk_swiglu", 1, 1, 300, 128, d_h=256, chunk=128, dtype="bf16"),
    workloads.make_spec("per_token_linear_exclusive", 1, 2, 300, 128, chunk=64, dtype="bf16"),
    workloads.make_spec("large_chunk_linear_update_first", 1, 2, 1000, 64, chunk=256, dtype="bf16"),
    workloads.make_spec("large_chunk_swiglu_last_layer", 1, 1, 300, 128, d_h=256, chunk=128, dtype="bf16"),
    workloads.make_spec("large_chunk_swiglu_last_layer", 1, 16, 300, 128, d_h=256, chunk=128, dtype="bf16"),
]


@pytest.mark.gpu
@pytest.mark.parametrize("s", CASES, ids=lambda s: f"{s['mode']}-{s['dtype']}")
def test_timed_matches_untimed(s):
    x = workloads.generate(s, seed=3)
    t = to_device(x, s)
    O1, W1 = la.forward(t["Q"], t["K"], t["V"], t["eta"], t["W0"], s["chunk"], s["mode"])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    O2, W2 = la.forward(t["Q"], t["K"], t["V"], t["eta"], t["W0"], s["chunk"], s["mode"], timing=(e0, e1))
    torch.cuda.synchronize()
    assert torch.equal(O1.view(torch.int16) if O1.dtype == torch.bfloat16 else O1,
                       O2.view(torch.int16) if O2.dtype == torch.bfloat16 else O2)
    assert torch.equal(W1, W2)
    ms = e0.elapsed_time(e1)
    print(f"[timed {s['mode']} {s['dtype']}] dominant kernel {ms * 1e3:.1f} us", flush=True)
    assert ms > 0


@pytest.mark.gpu
def test_fence_free_timing_events():
    """ttt_la_event_create/record/elapsed_ms: fence-free events passed to
    ttt_la_forward_timed bracket the dominant kernel, which lies inside an
    ordinary pair of events around the whole call."""
    s = CASES[0]
    x = workloads.generate(s, seed=5)
    t = to_device(x, s)
    O1, W1 = la.forward(t["Q"], t["K"], t["V"], t["eta"], t["W0"], s["chunk"], s["mode"])
    stream = torch.cuda.current_stream()
    k0, k1 = la.TimingEvent(), la.TimingEvent()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    O2, W2 = la.forward(t["Q"], t["K"], t["V"], t["eta"], t["W0"], s["chunk"], s["mode"], timing=(k0, k1))
    b.record(stream)
    torch.cuda.synchronize()
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16)) and torch.equal(W1, W2)
    kms, total = k0.elapsed_ms(k1), a.elapsed_time(b)
    print(f"[fence-free events] kernel {kms * 1e3:.1f} us of {total * 1e3:.1f} us", flush=True)
    assert 0 < kms <= total
