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
    (1, 1, 1100, 64, 64, "fp32"),      # fp32, 18 chunks: the sequential form (short sequences run a workgroup per chunk)
    (4, 16, 256, 64, 64, "fp32"),      # fp32, 128 head-column workgroups: the sequential form
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


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 64)])
def test_per_token_chunk_invariance(dtype, d):
    # fp32: the chunk is the kernel's tile, so the walk really changes.  bf16: the kernels tile by 64 tokens
    # whatever the chunk (the chunk is a tile length only), so this checks that the argument changes
    # nothing; the segment plan, which does change the computation, is varied by the segmentation test below
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



@pytest.mark.parametrize("B,H,T,d,mode", [
    (1, 2, 333, 128, "per_token_linear"),          # ragged tail, several segments
    (2, 3, 200, 64, "per_token_linear"),
    (1, 3, 150, 128, "per_token_linear_exclusive"),
    (1, 1, 1, 128, "per_token_linear"),            # single token
])
def test_per_token_float32_output(B, H, T, d, mode):
    s = workloads.make_spec(mode, B, H, T, d, chunk=64, dtype="bf16", eta="sigmoid", o_dtype="fp32")
    x = workloads.generate(s, seed=12)
    t = to_device(x, s)
    O32, W32 = run(t, s)
    assert O32.dtype == torch.float32
    check(s, x, O32, W32, label=f"{B},{H},{T},{d} float32 O")
    O16, W16 = run(t, dict(s, o_dtype="bf16"))
    # both write the same float32 accumulators; the bf16 output is their round-to-nearest-even
    assert torch.equal(O32.to(torch.bfloat16), O16)
    assert torch.equal(W32, W16)


@pytest.mark.parametrize("d", [128, 64])
def test_per_token_segmentation_invariance(d):
    # the segment plan depends on the number of heads: one head alone is cut into many segments, the
    # same head among 256 runs as one segment, among 16 as a few; outputs agree with the oracle and,
    # in float32, with each other to rounding
    T = 2048 if d == 128 else 4096      # (d = 64 fits two workgroups per CU: longer, to vary its plan too)
    s = workloads.make_spec("per_token_linear", 2, 128, T, d, chunk=64, dtype="bf16", eta="sigmoid", o_dtype="fp32")
    x = workloads.generate(s, seed=13)
    t = to_device(x, s)
    h = 37
    outs = {}
    for nh, sl in ((256, slice(None)), (16, slice(32, 48)), (1, slice(h, h + 1))):
        part = {k: v.reshape((256,) + tuple(v.shape[2:]))[sl].reshape((1, -1) + tuple(v.shape[2:])).contiguous()
                for k, v in t.items()}
        O, W = run(part, dict(s, B=1, H=nh))
        j = h if nh == 256 else (h - 32 if nh == 16 else 0)
        outs[nh] = (O[:, j:j + 1].cpu().numpy(), W[:, j:j + 1].cpu().numpy())
        plan = la.workspace_bytes(la.make_desc(1, nh, T, d, d, 0, la.BF16, la.O_FP32), 64, 0)
        print(f"heads {nh}: workspace {plan} bytes", flush=True)
    xs = {k: v.reshape((256,) + v.shape[2:])[h:h + 1][None] for k, v in x.items() if k in ("Q", "K", "V", "eta", "W0")}
    for nh, (O, W) in outs.items():
        check(dict(s, B=1, H=1), xs, torch.from_numpy(O), torch.from_numpy(W), label=f"head {h} among {nh}")
    for nh in (16, 1):
        assert err(outs[nh][0], outs[256][0], "bf16") <= 1e-4
        assert err(outs[nh][1], outs[256][1], "bf16") <= 1e-4


@pytest.mark.parametrize("B,H,T,mode", [
    (4, 16, 333, "per_token_linear"),              # 64 heads, ragged tail
    (4, 16, 64, "per_token_linear_exclusive"),     # one whole tile
    (4, 16, 1, "per_token_linear"),                # single token
    (2, 40, 130, "per_token_linear_exclusive"),    # 80 heads, 3 segments of one tile
    (3, 25, 200, "per_token_linear"),              # 75 heads, 2 segments
])
def test_per_token_many_heads(B, H, T, mode):
    # 64 to 255 heads of d = 128 with bf16 outputs: one to three segments per head (head counts that
    # are not powers of two in the last cases); the same heads in a batch of 8 are cut into one segment
    # per 64-token tile
    s = workloads.make_spec(mode, B, H, T, 128, chunk=64, dtype="bf16", eta="sigmoid")
    x = workloads.generate(s, seed=21)
    t = to_device(x, s)
    O, W = run(t, s)
    check(s, x, O, W, label=f"{B},{H},{T} {mode}")
    if mode == "per_token_linear_exclusive":
        _, Wi = run(t, dict(s, mode="per_token_linear"))
        assert torch.equal(W, Wi)
    # the first 8 heads alone reach the same final state to float32 rounding (their bf16
    # outputs may differ by an ulp, which for the largest entries is about 2% of the RMS)
    part = {k: v.reshape((B * H,) + tuple(v.shape[2:]))[:8].reshape((1, 8) + tuple(v.shape[2:])).contiguous()
            for k, v in t.items()}
    _, Ws = run(part, dict(s, B=1, H=8))
    Wc = W.reshape((B * H,) + tuple(W.shape[2:]))[:8].cpu().numpy()
    assert err(Ws[0].cpu().numpy(), Wc, "bf16") <= 1e-4
