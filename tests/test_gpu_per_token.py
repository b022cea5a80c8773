"""GPU parity of the per-token mode against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

from helpers import check, err, la, run, to_device, tol, workloads

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,H,T,d,chunk,dtype", [
    (1, 2, 256, 128, 64, "bf16"),
    (2, 3, 333, 128, 64, "bf16"),      # ragged tail, several tiles
    (1, 2, 777, 64, 64, "bf16"),
    (1, 4, 500, 128, 128, "bf16"),
    (2, 2, 300, 64, 128, "bf16"),
    (1, 1, 1, 128, 64, "bf16"),        # single token
    (1, 3, 150, 128, 32, "bf16"),
    (1, 3, 150, 64, 16, "bf16"),
    (1, 1, 256, 64, 64, "fp32"),
    (2, 2, 203, 128, 32, "fp32"),
    (1, 2, 90, 64, 16, "fp32"),
    (1, 2, 200, 128, 64, "fp32"),      # fp32, d = 128 with 64-token chunks, ragged
    (1, 1, 37, 64, 32, "fp32"),        # fp32, one partial chunk
])
def test_per_token_small(B, H, T, d, chunk, dtype):
    s = workloads.make_spec("per_token_linear", B, H, T, d, chunk=chunk, dtype=dtype, eta="sigmoid")
    x = workloads.generate(s, seed=1)
    O, W = run(to_device(x, s), s)
    check(s, x, O, W, label=f"{B},{H},{T},{d},c{chunk},{dtype}")


def test_per_token_empty_sequence():
    s = workloads.make_spec("per_token_linear", 1, 2, 0, 128, chunk=64, dtype="bf16")
    x = workloads.generate(s, seed=0)
    O, W = run(to_device(x, s), s)
    assert O.shape == (1, 2, 0, 128)
    assert torch.equal(W.cpu(), torch.from_numpy(x["W0"]))


def test_per_token_workload_fp32_full():
    s = workloads.spec("per_token_fp32_B1H1T256_d64_c64")
    x = workloads.generate(s, seed=0)
    O, W = run(to_device(x, s), s)
    check(s, x, O, W, label="fp32 B1H1T256")


def test_per_token_workload_B4H16T4096_sampled_heads():
    s = workloads.spec("per_token_bf16_B4H16T4096_d128_c64")
    x = workloads.generate(s, seed=0)
    O, W = run(to_device(x, s), s)
    check(s, x, O, W, heads=[0, 17, 38, 63], label="bf16 B4H16T4096 heads 0,17,38,63")


def test_per_token_workload_B1H32T32768_sampled_heads():
    s = workloads.spec("per_token_bf16_B1H32T32768_d128_c128")
    x = workloads.generate(s, seed=0)
    O, W = run(to_device(x, s), s)
    check(s, x, O, W, heads=[5, 31], label="bf16 B1H32T32768 heads 5,31")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 64)])
def test_per_token_chunk_invariance(dtype, d):
    s = workloads.make_spec("per_token_linear", 1, 4, 384, d, dtype=dtype, eta="sigmoid")
    x = workloads.generate(s, seed=3)
    t = to_device(x, s)
    chunks = [16, 32, 64, 128] if dtype == "bf16" else [16, 32, 64]
    outs = [run(t, s, chunk=c) for c in chunks]
    O0 = outs[0][0].float().cpu().numpy()
    for c, (O, W) in zip(chunks, outs):
        check(dict(s, chunk=c), x, O, W, label=f"chunk {c}")
        assert err(O.float().cpu().numpy(), O0, dtype) <= tol(dtype)


def test_per_token_deterministic_and_in_place():
    s = workloads.make_spec("per_token_linear", 2, 4, 700, 128, chunk=64, dtype="bf16", eta="sigmoid")
    x = workloads.generate(s, seed=4)
    t = to_device(x, s)
    O1, W1 = run(t, s)
    O2, W2 = run(t, s)
    assert torch.equal(O1, O2) and torch.equal(W1, W2)
    Wstate = t["W0"].clone()
    O3, W3 = la.forward(t["Q"], t["K"], t["V"], t["eta"], Wstate, 64, "per_token_linear", W_out=Wstate)
    torch.cuda.synchronize()
    assert W3.data_ptr() == Wstate.data_ptr()
    assert torch.equal(O3, O1) and torch.equal(W3, W1)


@pytest.mark.parametrize("t1", [64, 100])
def test_per_token_resume(t1):
    s = workloads.make_spec("per_token_linear", 1, 2, 300, 128, chunk=64, dtype="bf16", eta="sigmoid")
    x = workloads.generate(s, seed=5)
    t = to_device(x, s)
    O, W = run(t, s)
    a = {k: (v[:, :, :t1].contiguous() if k != "W0" else v) for k, v in t.items()}
    O1, Wm = run(a, s)
    b = {k: (v[:, :, t1:].contiguous() if k != "W0" else Wm) for k, v in t.items()}
    O2, W2 = run(b, s)
    Ocat = torch.cat([O1, O2], dim=2).float().cpu().numpy()
    assert err(Ocat, O.float().cpu().numpy(), "bf16") <= tol("bf16")
    assert err(W2.cpu().numpy(), W.cpu().numpy(), "bf16") <= tol("bf16")


def test_per_token_gradient_ascent_and_zero_rate():
    s = workloads.make_spec("per_token_linear", 1, 2, 200, 128, chunk=64, dtype="bf16", eta="normal", eta_scale=0.05)
    x = workloads.generate(s, seed=6)     # eta of both signs
    O, W = run(to_device(x, s), s)
    check(s, x, O, W, label="signed eta")
    x0 = dict(x, eta=np.zeros_like(x["eta"]))
    O, W = run(to_device(x0, s), s)
    check(s, x0, O, W, label="zero eta")
    assert torch.equal(W.cpu(), torch.from_numpy(x["W0"]))


@pytest.mark.parametrize("B,H,T,d,chunk,dtype", [
    (1, 2, 256, 128, 64, "bf16"),
    (2, 3, 333, 128, 64, "bf16"),      # ragged tail, several segments
    (1, 1, 300, 64, 64, "bf16"),       # five one-tile segments
    (1, 3, 150, 64, 16, "bf16"),
    (1, 4, 500, 128, 128, "bf16"),
    (1, 1, 1, 128, 64, "bf16"),        # single token: its output is W0's read
    (1, 1, 256, 64, 64, "fp32"),
    (2, 2, 203, 128, 32, "fp32"),
    (1, 1, 37, 64, 32, "fp32"),
])
def test_per_token_exclusive_small(B, H, T, d, chunk, dtype):
    s = workloads.make_spec("per_token_linear_exclusive", B, H, T, d, chunk=chunk, dtype=dtype, eta="sigmoid")
    x = workloads.generate(s, seed=7)
    t = to_device(x, s)
    O, W = run(t, s)
    check(s, x, O, W, label=f"{B},{H},{T},{d},c{chunk},{dtype}")
    # the read order does not touch the state sequence: same kernels, same final state
    _, Wi = run(t, dict(s, mode="per_token_linear"))
    assert torch.equal(W, Wi)


def test_per_token_exclusive_workload_B4H16T4096_sampled_heads():
    s = workloads.spec("per_token_bf16_B4H16T4096_d128_c64", mode="per_token_linear_exclusive")
    x = workloads.generate(s, seed=0)
    O, W = run(to_device(x, s), s)
    check(s, x, O, W, heads=[0, 17, 38, 63], label="bf16 B4H16T4096 heads 0,17,38,63")
