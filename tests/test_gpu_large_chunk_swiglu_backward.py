"""GPU parity of the SwiGLU backward (ttt_la_backward in the three SwiGLU
modes) against the fp64 oracle: dQ, dK, dV, deta and dW0, each within
2e-2 of its RMS (the gradients are float32)."""
import numpy as np
import pytest
import torch

from helpers import la, oracle, to_device, workloads

pytestmark = pytest.mark.gpu


def run_and_check(s, seed, label, tol=2e-2):
    x = workloads.generate(s, seed=seed)
    gr = workloads.generate_grads(s, seed=seed)
    t = to_device(x, s)
    dO = torch.from_numpy(gr["dO"]).cuda().to(torch.bfloat16)
    dW = torch.from_numpy(gr["dW"]).cuda()
    got = la.backward(t["Q"], t["K"], t["V"], t["eta"], t["W0"], dO, dW, s["chunk"], s["mode"])
    torch.cuda.synchronize()
    ref = oracle.backward(x["Q"], x["K"], x["V"], x["eta"], x["W0"], gr["dO"], gr["dW"], s["chunk"], s["mode"],
                          d_h=s["d_h"])
    errs = []
    for name, g, r in zip(("dQ", "dK", "dV", "deta", "dW0"), got, ref):
        g = g.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(g)), name
        rms = np.sqrt(np.mean(r * r)) if r.size else 1.0
        errs.append(np.abs(g - r).max() / max(rms, 1e-300) if r.size else 0.0)
    print(f"[{s['mode']} backward {label}] " + " ".join(f"{n}={e:.2e}" for n, e in
                                                        zip(("dQ", "dK", "dV", "deta", "dW0"), errs)), flush=True)
    assert max(errs) <= tol
    return got


MODES = ["large_chunk_swiglu", "large_chunk_swiglu_update_first", "large_chunk_swiglu_last_layer"]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("B,H,T,chunk", [
    (1, 1, 300, 128),      # ragged last chunk
    (1, 2, 700, 256),
    (2, 1, 200, 37),       # chunk not a multiple of the GEMM tiles
    (1, 1, 100, 2048),     # one chunk, shorter than its length
    (1, 1, 48, 4),         # many tiny chunks
])
def test_swiglu_backward_small(mode, B, H, T, chunk):
    s = workloads.make_spec(mode, B, H, T, 128, d_h=256, chunk=chunk, dtype="bf16", eta_scale=0.02)
    run_and_check(s, 50, f"{B},{H},{T},c{chunk}")


def test_swiglu_backward_more_heads_than_one_launch():
    s = workloads.make_spec("large_chunk_swiglu", 2, 9, 300, 128, d_h=256, chunk=128, dtype="bf16", eta_scale=0.02)
    run_and_check(s, 51, "2x9 heads")


def test_swiglu_backward_empty_and_deterministic():
    s = workloads.make_spec("large_chunk_swiglu", 1, 2, 0, 128, d_h=256, chunk=128, dtype="bf16")
    x = workloads.generate(s, seed=0)
    gr = workloads.generate_grads(s, seed=0)
    t = to_device(x, s)
    dO = torch.from_numpy(gr["dO"]).cuda().to(torch.bfloat16)
    dW = torch.from_numpy(gr["dW"]).cuda()
    got = la.backward(t["Q"], t["K"], t["V"], t["eta"], t["W0"], dO, dW, 128, s["mode"])
    torch.cuda.synchronize()
    assert torch.equal(got[4], dW)
    s = workloads.make_spec("large_chunk_swiglu", 1, 2, 500, 128, d_h=256, chunk=128, dtype="bf16", eta_scale=0.02)
    x = workloads.generate(s, seed=52)
    gr = workloads.generate_grads(s, seed=52)
    t = to_device(x, s)
    dO = torch.from_numpy(gr["dO"]).cuda().to(torch.bfloat16)
    dW = torch.from_numpy(gr["dW"]).cuda()
    a = la.backward(t["Q"], t["K"], t["V"], t["eta"], t["W0"], dO, dW, 128, s["mode"])
    b = la.backward(t["Q"], t["K"], t["V"], t["eta"], t["W0"], dO, dW, 128, s["mode"])
    torch.cuda.synchronize()
    assert all(torch.equal(u, v) for u, v in zip(a, b))


@pytest.mark.parametrize("mode", MODES)
def test_swiglu_backward_workload_all_heads(mode):
    s = workloads.spec("large_chunk_swiglu_bf16_B2H8T32768_d128_dh256_c2048", mode=mode)
    run_and_check(s, 0, "B2H8T32768 all heads")
