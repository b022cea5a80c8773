"""GPU parity of the large-chunk (LaCT) linear mode against the fp64 oracle."""
import numpy as np
import pytest
import torch

from helpers import check, err, la, run, to_device, tol, workloads

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,H,T,d,chunk", [
    (1, 2, 300, 64, 128),     # ragged last chunk
    (2, 2, 512, 64, 256),
    (1, 3, 1000, 128, 300),   # chunk not a multiple of the tiles
    (1, 1, 2500, 64, 2048),   # several token slices per chunk, ragged
    (1, 2, 97, 64, 1),        # one token per chunk
    (1, 2, 50, 64, 7),
    (1, 2, 100, 64, 100),     # a single chunk
    (1, 2, 100, 64, 4096),    # chunk longer than the sequence
    (1, 2, 700, 128, 32),     # d = 128 over several scan windows of chunks, ragged
    (1, 1, 1500, 64, 50),     # d = 64 over three scan windows, the last one partial
])
def test_large_chunk_linear_small(B, H, T, d, chunk):
    s = workloads.make_spec("large_chunk_linear", B, H, T, d, chunk=chunk, dtype="bf16", eta_scale=0.05)
    x = workloads.generate(s, seed=2)
    O, W = run(to_device(x, s), s)
    check(s, x, O, W, label=f"{B},{H},{T},{d},c{chunk}")
    assert np.allclose(np.linalg.norm(W.cpu().numpy().astype(np.float64), axis=-2), 1.0, atol=1e-5)


def test_large_chunk_linear_empty():
    s = workloads.make_spec("large_chunk_linear", 1, 2, 0, 64, chunk=64, dtype="bf16")
    x = workloads.generate(s, seed=0)
    O, W = run(to_device(x, s), s)
    assert torch.equal(W.cpu(), torch.from_numpy(x["W0"]))


def test_large_chunk_linear_deterministic_resume_in_place():
    s = workloads.make_spec("large_chunk_linear", 1, 3, 700, 64, chunk=128, dtype="bf16", eta_scale=0.05)
    x = workloads.generate(s, seed=3)
    t = to_device(x, s)
    O1, W1 = run(t, s)
    O2, W2 = run(t, s)
    assert torch.equal(O1, O2) and torch.equal(W1, W2)
    t1 = 256                          # a chunk boundary
    a = {k: (v[:, :, :t1].contiguous() if k != "W0" else v) for k, v in t.items()}
    Oa, Wm = run(a, s)
    b = {k: (v[:, :, t1:].contiguous() if k != "W0" else Wm) for k, v in t.items()}
    Ob, Wb = run(b, s)
    assert err(torch.cat([Oa, Ob], 2).float().cpu().numpy(), O1.float().cpu().numpy(), "bf16") <= tol("bf16")
    assert err(Wb.cpu().numpy(), W1.cpu().numpy(), "bf16") <= tol("bf16")
    Ws = t["W0"].clone()
    O3, W3 = la.forward(t["Q"], t["K"], t["V"], t["eta"], Ws, 128, "large_chunk_linear", W_out=Ws)
    torch.cuda.synchronize()
    assert torch.equal(O3, O1) and torch.equal(W3, W1)


@pytest.mark.parametrize("B,H,T,d,chunk", [
    (1, 2, 300, 64, 128),     # ragged last chunk
    (1, 3, 1000, 128, 300),
    (1, 1, 2500, 64, 2048),   # several token slices per chunk
    (1, 2, 97, 64, 1),        # one token per chunk
    (1, 2, 100, 64, 4096),    # a single chunk
    (1, 2, 700, 128, 32),     # several scan windows
])
def test_large_chunk_linear_update_first_small(B, H, T, d, chunk):
    s = workloads.make_spec("large_chunk_linear_update_first", B, H, T, d, chunk=chunk, dtype="bf16",
                            eta_scale=0.05)
    x = workloads.generate(s, seed=8)
    t = to_device(x, s)
    O, W = run(t, s)
    check(s, x, O, W, label=f"{B},{H},{T},{d},c{chunk}")
    _, Wr = run(t, dict(s, mode="large_chunk_linear"))
    assert torch.equal(W, Wr)


def momentum_check(s, x, O, W, M, beta, M0=None, label=""):
    import oracle
    Or, Wr, Mr = oracle.large_chunk_linear(x["Q"], x["K"], x["V"], x["eta"], x["W0"], s["chunk"],
                                           read_first=s["mode"] == "large_chunk_linear", momentum=beta, M0=M0)
    eo, ew, em = (err(O.float().cpu().numpy(), Or, "bf16"), err(W.cpu().numpy(), Wr, "bf16"),
                  err(M.cpu().numpy(), Mr, "bf16"))
    print(f"[{s['mode']} momentum {beta} {label}] err_O={eo:.3e} err_W={ew:.3e} err_M={em:.3e}", flush=True)
    assert max(eo, ew, em) <= tol("bf16")


@pytest.mark.parametrize("mode", ["large_chunk_linear", "large_chunk_linear_update_first"])
@pytest.mark.parametrize("B,H,T,d,chunk,beta", [
    (1, 2, 300, 64, 128, 0.9),
    (1, 3, 1000, 128, 300, 0.5),
    (1, 2, 97, 64, 1, 0.9),        # one token per chunk: many momentum steps
    (1, 1, 2500, 64, 2048, -0.3),
])
def test_large_chunk_linear_momentum(mode, B, H, T, d, chunk, beta):
    s = workloads.make_spec(mode, B, H, T, d, chunk=chunk, dtype="bf16", eta_scale=0.05)
    x = workloads.generate(s, seed=23)
    t = to_device(x, s)
    O, W, M = la.forward_momentum(t["Q"], t["K"], t["V"], t["eta"], t["W0"], chunk, beta, mode=mode)
    torch.cuda.synchronize()
    momentum_check(s, x, O, W, M, beta, label=f"{B},{H},{T},{d},c{chunk}")


def test_large_chunk_linear_momentum_zero_is_forward_and_resume():
    s = workloads.make_spec("large_chunk_linear", 1, 3, 700, 64, chunk=128, dtype="bf16", eta_scale=0.05)
    x = workloads.generate(s, seed=24)
    t = to_device(x, s)
    O0, W0_ = run(t, s)
    Om, Wm, _ = la.forward_momentum(t["Q"], t["K"], t["V"], t["eta"], t["W0"], 128, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(O0, Om) and torch.equal(W0_, Wm)          # momentum 0 is the plain method, bit for bit
    O, W, M = la.forward_momentum(t["Q"], t["K"], t["V"], t["eta"], t["W0"], 128, 0.8)
    a = {k: (v[:, :, :256].contiguous() if k != "W0" else v) for k, v in t.items()}
    b = {k: (v[:, :, 256:].contiguous() if k != "W0" else v) for k, v in t.items()}
    Oa, Wa, Ma = la.forward_momentum(a["Q"], a["K"], a["V"], a["eta"], a["W0"], 128, 0.8)
    Ob, Wb, Mb = la.forward_momentum(b["Q"], b["K"], b["V"], b["eta"], Wa, 128, 0.8, M0=Ma)
    torch.cuda.synchronize()
    assert err(torch.cat([Oa, Ob], 2).float().cpu().numpy(), O.float().cpu().numpy(), "bf16") <= tol("bf16")
    assert err(Wb.cpu().numpy(), W.cpu().numpy(), "bf16") <= 1e-5 and err(Mb.cpu().numpy(), M.cpu().numpy(), "bf16") <= 1e-5


def test_large_chunk_linear_momentum_workload_all_heads():
    s = workloads.spec("large_chunk_linear_bf16_B1H12T196608_d64_c4096")
    x = workloads.generate(s, seed=0)
    t = to_device(x, s)
    O, W, M = la.forward_momentum(t["Q"], t["K"], t["V"], t["eta"], t["W0"], s["chunk"], 0.9)
    torch.cuda.synchronize()
    del t
    momentum_check(dict(s), x, O, W, M, 0.9, label="B1H12T196608 all heads")


def test_large_chunk_linear_momentum_in_place_buffer():
    # M_out == M0: the buffer is updated in place, as two calls on the halves of the sequence show
    s = workloads.make_spec("large_chunk_linear", 1, 2, 512, 64, chunk=128, dtype="bf16", eta_scale=0.05)
    x = workloads.generate(s, seed=25)
    t = to_device(x, s)
    O, W, M = la.forward_momentum(t["Q"], t["K"], t["V"], t["eta"], t["W0"], 128, 0.7)
    desc = la.make_desc(1, 2, 256, 64, 64, 0, la.BF16)
    ws = torch.empty(max(la.workspace_bytes(desc, 128, 1), 1), dtype=torch.uint8, device="cuda")
    Mbuf = torch.zeros_like(t["W0"])
    Wcur = t["W0"].clone()
    outs = []
    for h in (slice(0, 256), slice(256, 512)):
        part = {k: t[k][:, :, h].contiguous() for k in ("Q", "K", "V", "eta")}
        Oh = torch.empty((1, 2, 256, 64), dtype=torch.bfloat16, device="cuda")
        st = la.forward_momentum_raw(part["Q"].data_ptr(), part["K"].data_ptr(), part["V"].data_ptr(),
                                     part["eta"].data_ptr(), Wcur.data_ptr(), Mbuf.data_ptr(), 0.7, 128, 1, desc,
                                     Oh.data_ptr(), Wcur.data_ptr(), Mbuf.data_ptr(), ws.data_ptr(), ws.numel(),
                                     torch.cuda.current_stream().cuda_stream)
        assert st == 0
        outs.append(Oh)
    torch.cuda.synchronize()
    assert err(torch.cat(outs, 2).float().cpu().numpy(), O.float().cpu().numpy(), "bf16") <= tol("bf16")
    assert err(Wcur.cpu().numpy(), W.cpu().numpy(), "bf16") <= 1e-5
    assert err(Mbuf.cpu().numpy(), M.cpu().numpy(), "bf16") <= 1e-5


@pytest.mark.parametrize("B,H,T,d,chunk,mode", [
    (1, 2, 300, 64, 128, "large_chunk_linear"),
    (1, 3, 1000, 128, 300, "large_chunk_linear"),
    (1, 2, 97, 64, 1, "large_chunk_linear_update_first"),
    (1, 1, 2500, 64, 2048, "large_chunk_linear_update_first"),
])
def test_large_chunk_linear_float32_output(B, H, T, d, chunk, mode):
    s = workloads.make_spec(mode, B, H, T, d, chunk=chunk, dtype="bf16", eta_scale=0.05, o_dtype="fp32")
    x = workloads.generate(s, seed=14)
    t = to_device(x, s)
    O32, W32 = run(t, s)
    assert O32.dtype == torch.float32
    check(s, x, O32, W32, label=f"{B},{H},{T},{d},c{chunk} float32 O")
    O16, W16 = run(t, dict(s, o_dtype="bf16"))
    assert torch.equal(O32.to(torch.bfloat16), O16)
    assert torch.equal(W32, W16)
    Om, Wm, _ = la.forward_momentum(t["Q"], t["K"], t["V"], t["eta"], t["W0"], chunk, 0.0, mode=mode,
                                    out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(Om, O32) and torch.equal(Wm, W32)
