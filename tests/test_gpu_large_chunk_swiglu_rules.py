"""GPU parity of the SwiGLU memory's other update rules against the fp64
oracle: momentum (ttt_la_forward_momentum) and Muon (ttt_la_forward_muon),
with and without momentum, in both read orders."""
import numpy as np
import pytest
import torch

from helpers import err, la, to_device, tol, workloads
from oracle import large_chunk_swiglu, swiglu_pack, swiglu_unpack

pytestmark = pytest.mark.gpu

D, DH = 128, 256


def oracle_rule(x, s, beta=None, muon=None, M0=None):
    W1, W3, W2 = swiglu_unpack(x["W0"].astype(np.float64), D, DH)
    kw = dict(read_first=s["mode"] == "large_chunk_swiglu")
    if beta is not None:
        kw["momentum"] = beta
        if M0 is not None:
            kw["M0"] = swiglu_unpack(M0.astype(np.float64), D, DH)
    if muon is not None:
        kw["muon_scale"] = muon
    res = large_chunk_swiglu(x["Q"], x["K"], x["V"], x["eta"], W1, W3, W2, s["chunk"], **kw)
    M = swiglu_pack(*res[2]) if beta is not None else None
    return res[0], swiglu_pack(*res[1]), M


def check_rule(s, x, O, W, M, beta=None, muon=None, M0=None, label=""):
    Or, Wr, Mr = oracle_rule(x, s, beta, muon, M0)
    eo = err(O.float().cpu().numpy(), Or, "bf16")
    ew = err(W.cpu().numpy(), Wr, "bf16")
    # The momentum buffer is an increment of the weights: its error is taken on their scale, max|dM| over
    # RMS(W).  (On its own scale it shows the bf16 operands of the gradient products, about 2^-8 of each
    # chunk step, times the heavy tail of the buffer.)
    em, em_own = 0.0, 0.0
    if Mr is not None:
        dM = np.abs(M.cpu().numpy().astype(np.float64) - Mr).max()
        em = dM / np.sqrt(np.mean(Wr ** 2))
        em_own = err(M.cpu().numpy(), Mr, "bf16")
    print(f"[{s['mode']} beta={beta} muon={muon} {label}] err_O={eo:.3e} err_W={ew:.3e} err_M={em:.3e} "
          f"(on M's own RMS {em_own:.3e})", flush=True)
    assert eo <= tol("bf16") and ew <= tol("bf16") and em <= tol("bf16")
    W1, W3, W2 = swiglu_unpack(W.cpu().numpy().astype(np.float64), D, DH)
    for Wm in (W1, W3, W2):                     # the normalisation follows every rule
        assert np.allclose(np.linalg.norm(Wm, axis=-2), 1.0, atol=1e-5)


def spec(mode, B, H, T, chunk, seed_scale=0.02):
    return workloads.make_spec(mode, B, H, T, D, d_h=DH, chunk=chunk, dtype="bf16", eta_scale=seed_scale)


@pytest.mark.parametrize("B,H,T,chunk,mode,beta", [
    (1, 1, 300, 128, "large_chunk_swiglu", 0.9),           # ragged last chunk
    (1, 2, 1024, 256, "large_chunk_swiglu", 0.5),
    (2, 1, 700, 2048, "large_chunk_swiglu", 0.9),          # one chunk
    (1, 1, 200, 37, "large_chunk_swiglu_update_first", 0.8),
    (1, 1, 40, 1, "large_chunk_swiglu", 0.9),               # one token per chunk
])
def test_swiglu_momentum_small(B, H, T, chunk, mode, beta):
    s = spec(mode, B, H, T, chunk)
    x = workloads.generate(s, seed=40)
    t = to_device(x, s)
    O, W, M = la.forward_momentum(t["Q"], t["K"], t["V"], t["eta"], t["W0"], chunk, beta, mode=mode)
    torch.cuda.synchronize()
    check_rule(s, x, O, W, M, beta=beta, label=f"{B},{H},{T},c{chunk}")


def test_swiglu_momentum_zero_is_plain_descent_bit_for_bit():
    s = spec("large_chunk_swiglu", 1, 2, 700, 128)
    x = workloads.generate(s, seed=41)
    t = to_device(x, s)
    O0, W0_ = la.forward(t["Q"], t["K"], t["V"], t["eta"], t["W0"], 128, s["mode"])
    O, W, M = la.forward_momentum(t["Q"], t["K"], t["V"], t["eta"], t["W0"], 128, 0.0, mode=s["mode"])
    torch.cuda.synchronize()
    assert torch.equal(O.view(torch.int16), O0.view(torch.int16)) and torch.equal(W, W0_)


def test_swiglu_momentum_resume_and_empty():
    s = spec("large_chunk_swiglu", 1, 2, 512, 128)
    x = workloads.generate(s, seed=42)
    t = to_device(x, s)
    O, W, M = la.forward_momentum(t["Q"], t["K"], t["V"], t["eta"], t["W0"], 128, 0.7, mode=s["mode"])
    a = {k: (v[:, :, :256].contiguous() if k != "W0" else v) for k, v in t.items()}
    b = {k: (v[:, :, 256:].contiguous() if k != "W0" else v) for k, v in t.items()}
    Oa, Wa, Ma = la.forward_momentum(a["Q"], a["K"], a["V"], a["eta"], a["W0"], 128, 0.7, mode=s["mode"])
    Ob, Wb, Mb = la.forward_momentum(b["Q"], b["K"], b["V"], b["eta"], Wa, 128, 0.7, M0=Ma, mode=s["mode"])
    torch.cuda.synchronize()
    assert err(torch.cat([Oa, Ob], 2).float().cpu().numpy(), O.float().cpu().numpy(), "bf16") <= tol("bf16")
    assert err(Wb.cpu().numpy(), W.cpu().numpy(), "bf16") <= 1e-5
    assert err(Mb.cpu().numpy(), M.cpu().numpy(), "bf16") <= 1e-5
    # no tokens: the buffer passes through
    e = {k: (v[:, :, :0].contiguous() if k != "W0" else v) for k, v in t.items()}
    Oe, We, Me = la.forward_momentum(e["Q"], e["K"], e["V"], e["eta"], e["W0"], 128, 0.7, M0=M, mode=s["mode"])
    torch.cuda.synchronize()
    assert torch.equal(We, t["W0"]) and torch.equal(Me, M)


@pytest.mark.parametrize("B,H,T,chunk,mode,scale,beta", [
    (1, 1, 300, 128, "large_chunk_swiglu", 0.05, None),     # ragged last chunk
    (1, 2, 1024, 256, "large_chunk_swiglu", 0.1, None),
    (2, 1, 700, 2048, "large_chunk_swiglu", 0.05, None),    # one chunk
    (1, 1, 200, 37, "large_chunk_swiglu_update_first", 0.05, None),
    (1, 1, 600, 128, "large_chunk_swiglu", 0.05, 0.9),      # with momentum
    (1, 2, 500, 100, "large_chunk_swiglu_update_first", 0.02, 0.5),
    (1, 1, 40, 4, "large_chunk_swiglu", 0.05, None),        # four tokens per chunk: rank-4 steps
])
def test_swiglu_muon_small(B, H, T, chunk, mode, scale, beta):
    s = spec(mode, B, H, T, chunk)
    x = workloads.generate(s, seed=43)
    t = to_device(x, s)
    O, W, M = la.forward_muon(t["Q"], t["K"], t["V"], t["eta"], t["W0"], chunk, scale, momentum=beta or 0.0,
                              mode=mode)
    torch.cuda.synchronize()
    assert (M is None) == (beta is None)
    check_rule(s, x, O, W, M, beta=beta, muon=scale, label=f"{B},{H},{T},c{chunk}")


def test_swiglu_muon_more_heads_than_one_launch():
    # 18 heads: 16 in the first launch, 2 in the second, each with its own exchange region
    s = workloads.make_spec("large_chunk_swiglu", 2, 9, 300, D, d_h=DH, chunk=128, dtype="bf16", eta_scale=0.02,
                            o_dtype="fp32")
    x = workloads.generate(s, seed=44)
    t = to_device(x, s)
    O, W, M = la.forward_muon(t["Q"], t["K"], t["V"], t["eta"], t["W0"], 128, 0.05, momentum=0.9,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_rule(s, x, O, W, M, beta=0.9, muon=0.05, label="2x9 heads")


def test_swiglu_muon_deterministic():
    s = spec("large_chunk_swiglu", 1, 2, 700, 128)
    x = workloads.generate(s, seed=45)
    t = to_device(x, s)
    r1 = la.forward_muon(t["Q"], t["K"], t["V"], t["eta"], t["W0"], 128, 0.05, momentum=0.5)
    r2 = la.forward_muon(t["Q"], t["K"], t["V"], t["eta"], t["W0"], 128, 0.05, momentum=0.5)
    torch.cuda.synchronize()
    assert all(torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b) for a, b in zip(r1, r2))


@pytest.mark.parametrize("rule", ["momentum", "muon", "muon_momentum"])
def test_swiglu_rules_workload_all_heads(rule):
    # O in float32: with momentum the weights' trajectory moves by a few 1e-3 of their RMS under the bf16
    # operands of the gradient products (emulated in fp64: uniformly over heads), which on top of a bf16
    # output's own rounding (1.6e-2 of RMS here) would leave no margin
    s = workloads.spec("large_chunk_swiglu_bf16_B2H8T32768_d128_dh256_c2048")
    x = workloads.generate(s, seed=0)
    t = to_device(x, s)
    f32 = torch.float32
    if rule == "momentum":
        O, W, M = la.forward_momentum(t["Q"], t["K"], t["V"], t["eta"], t["W0"], s["chunk"], 0.9, mode=s["mode"],
                                      out_dtype=f32)
        beta, scale = 0.9, None
    else:
        beta = 0.9 if rule == "muon_momentum" else None
        O, W, M = la.forward_muon(t["Q"], t["K"], t["V"], t["eta"], t["W0"], s["chunk"], 0.05,
                                  momentum=beta or 0.0, out_dtype=f32)
        scale = 0.05
    torch.cuda.synchronize()
    del t
    check_rule(s, x, O, W, M, beta=beta, muon=scale, label="B2H8T32768 all heads")
