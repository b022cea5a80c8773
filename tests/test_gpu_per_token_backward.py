"""GPU parity of the per-token backward against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

from helpers import err, gpu_heads, la, oracle, tol, to_device, workloads

pytestmark = pytest.mark.gpu

NAMES = ("dQ", "dK", "dV", "deta", "dW0")


def run_backward(t, g, s):
    out = la.backward(t["Q"], t["K"], t["V"], t["eta"], t["W0"], g["dO"], g["dW"], s["chunk"], s["mode"])
    torch.cuda.synchronize()
    return out


def grads_to_device(gr, dev="cuda", dtype=torch.bfloat16):
    return dict(dO=torch.from_numpy(gr["dO"]).to(dev).to(dtype), dW=torch.from_numpy(gr["dW"]).to(dev))


def check_backward(s, x, gr, out, heads=None, label=""):
    def sel(a):
        if heads is None:
            return a
        B, H = a.shape[:2]
        return a.reshape((B * H,) + a.shape[2:])[heads][None]
    ref = oracle.backward(sel(x["Q"]), sel(x["K"]), sel(x["V"]), sel(x["eta"]), sel(x["W0"]), sel(gr["dO"]),
                          sel(gr["dW"]), s["chunk"], s["mode"])
    dt = s["dtype"]
    errs = {n: err(gpu_heads(o, heads), r, dt) for n, o, r in zip(NAMES, out, ref)}
    print(f"[{s['mode']} backward {label} {dt}] " + " ".join(f"{n}={e:.3e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= tol(dt), f"{n} error {e} > {tol(dt)}"


@pytest.mark.parametrize("mode", ["per_token_linear", "per_token_linear_exclusive"])
@pytest.mark.parametrize("B,H,T,d,chunk", [
    (1, 2, 256, 128, 64),
    (2, 3, 333, 128, 64),      # ragged tail, several segments
    (1, 1, 300, 64, 64),       # five one-tile segments, the last partial
    (1, 2, 777, 64, 32),
    (1, 3, 150, 128, 128),
    (1, 1, 1, 128, 64),        # single token
    (1, 2, 64, 64, 16),        # one full tile
])
def test_per_token_backward_small(mode, B, H, T, d, chunk):
    s = workloads.make_spec(mode, B, H, T, d, chunk=chunk, dtype="bf16", eta="sigmoid")
    x = workloads.generate(s, seed=11)
    gr = workloads.generate_grads(s, seed=11)
    out = run_backward(to_device(x, s), grads_to_device(gr), s)
    check_backward(s, x, gr, out, label=f"{B},{H},{T},{d},c{chunk}")


def test_per_token_backward_empty_sequence():
    s = workloads.make_spec("per_token_linear", 1, 2, 0, 128, chunk=64, dtype="bf16")
    x = workloads.generate(s, seed=0)
    gr = workloads.generate_grads(s, seed=0)
    dQ, dK, dV, deta, dW0 = run_backward(to_device(x, s), grads_to_device(gr), s)
    assert dQ.shape == (1, 2, 0, 128) and deta.shape == (1, 2, 0)
    assert torch.equal(dW0.cpu(), torch.from_numpy(gr["dW"]))


def test_per_token_backward_signed_and_zero_rates():
    s = workloads.make_spec("per_token_linear", 1, 2, 200, 128, chunk=64, dtype="bf16", eta="normal", eta_scale=0.05)
    x = workloads.generate(s, seed=12)
    gr = workloads.generate_grads(s, seed=12)
    out = run_backward(to_device(x, s), grads_to_device(gr), s)
    check_backward(s, x, gr, out, label="signed eta")
    x0 = dict(x, eta=np.zeros_like(x["eta"]))
    dQ, dK, dV, deta, dW0 = run_backward(to_device(x0, s), grads_to_device(gr), s)
    assert not dK.any() and not dV.any()        # no step, so no gradient reaches K or V
    check_backward(s, x0, gr, (dQ, dK, dV, deta, dW0), label="zero eta")


def test_per_token_backward_deterministic():
    s = workloads.make_spec("per_token_linear", 2, 4, 700, 128, chunk=64, dtype="bf16", eta="sigmoid")
    x = workloads.generate(s, seed=13)
    gr = workloads.generate_grads(s, seed=13)
    t, g = to_device(x, s), grads_to_device(gr)
    a = run_backward(t, g, s)
    b = run_backward(t, g, s)
    assert all(torch.equal(u, v) for u, v in zip(a, b))


def test_per_token_backward_workload_B4H16T4096_sampled_heads():
    s = workloads.spec("per_token_bf16_B4H16T4096_d128_c64")
    x = workloads.generate(s, seed=0)
    gr = workloads.generate_grads(s, seed=0)
    out = run_backward(to_device(x, s), grads_to_device(gr), s)
    check_backward(s, x, gr, out, heads=[0, 21, 63], label="B4H16T4096 heads 0,21,63")


@pytest.mark.parametrize("mode", ["per_token_linear", "per_token_linear_exclusive"])
@pytest.mark.parametrize("B,H,T,d,chunk", [
    (1, 1, 256, 64, 64),
    (2, 2, 203, 128, 32),      # ragged tail
    (1, 2, 90, 64, 16),
    (1, 1, 1, 64, 64),         # single token
    (1, 1, 1100, 64, 64),      # 18 chunks: the sequential form of the float32 kernel
])
def test_per_token_backward_fp32(mode, B, H, T, d, chunk):
    s = workloads.make_spec(mode, B, H, T, d, chunk=chunk, dtype="fp32", eta="sigmoid")
    x = workloads.generate(s, seed=14)
    gr = workloads.generate_grads(s, seed=14)
    out = run_backward(to_device(x, s), grads_to_device(gr, dtype=torch.float32), s)
    check_backward(s, x, gr, out, label=f"{B},{H},{T},{d},c{chunk}")


def test_per_token_backward_workload_fp32_full():
    s = workloads.spec("per_token_fp32_B1H1T256_d64_c64")
    x = workloads.generate(s, seed=0)
    gr = workloads.generate_grads(s, seed=0)
    out = run_backward(to_device(x, s), grads_to_device(gr, dtype=torch.float32), s)
    check_backward(s, x, gr, out, label="fp32 B1H1T256")
