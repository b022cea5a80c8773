"""Shared helpers for the GPU parity tests (imports torch and the binding)."""
import os

import numpy as np
import torch

import linear_attention_ttt_amd as la
import oracle
import workloads

FP32_TOL = 1e-4      # max |o - r| / max |r|   (float32 inputs)
BF16_TOL = 2e-2      # max |o - r| / RMS(r)    (bfloat16 inputs)


def to_device(x, s, dev="cuda"):
    dt = torch.bfloat16 if s["dtype"] == "bf16" else torch.float32
    t = {k: torch.from_numpy(np.ascontiguousarray(x[k])).to(dev) for k in ("Q", "K", "V", "eta", "W0")}
    for k in ("Q", "K", "V"):
        t[k] = t[k].to(dt)
    return t


def out_dtype(s):
    """torch dtype of O for workload parameters ``s``."""
    return torch.float32 if s.get("o_dtype", s["dtype"]) == "fp32" else torch.bfloat16


def run(t, s, chunk=None, **kw):
    kw.setdefault("out_dtype", out_dtype(s))
    O, W = la.forward(t["Q"], t["K"], t["V"], t["eta"], t["W0"], s["chunk"] if chunk is None else chunk,
                      s["mode"], **kw)
    torch.cuda.synchronize()
    return O, W


def err(got, ref, dtype):
    """Error metric of the accuracy bound for this input dtype."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    d = np.abs(got - ref).max()
    if dtype == "fp32":
        return d / max(np.abs(ref).max(), 1e-300)
    return d / max(np.sqrt(np.mean(ref ** 2)), 1e-300)


def tol(dtype):
    return FP32_TOL if dtype == "fp32" else BF16_TOL


def oracle_heads(x, s, heads=None):
    """Oracle on a subset of (flattened) heads; returns (O, W) for those."""
    def sel(a):
        if heads is None:
            return a
        B, H = a.shape[:2]
        flat = a.reshape((B * H,) + a.shape[2:])[heads]
        return flat[None]
    return oracle.forward(sel(x["Q"]), sel(x["K"]), sel(x["V"]), sel(x["eta"]), sel(x["W0"]), s["chunk"],
                          s["mode"], d_h=s["d_h"])


def gpu_heads(T_, heads):
    a = T_.float().cpu().numpy() if T_.dtype != torch.float32 else T_.cpu().numpy()
    if heads is None:
        return a
    B, H = a.shape[:2]
    return a.reshape((B * H,) + a.shape[2:])[heads][None]


def check(s, x, O, W, heads=None, label=""):
    Or, Wr = oracle_heads(x, s, heads)
    eo = err(gpu_heads(O, heads), Or, s["dtype"])
    ew = err(gpu_heads(W, heads), Wr, s["dtype"])
    line = f"[{s['mode']} {label}] err_O={eo:.3e} err_W={ew:.3e} tol={tol(s['dtype'])}"
    print(line, flush=True)
    if os.environ.get("TTT_ERRLOG"):
        with open(os.environ["TTT_ERRLOG"], "a") as f:
            f.write(line + "\n")
    assert eo <= tol(s["dtype"]), f"O error {eo} > {tol(s['dtype'])}"
    assert ew <= tol(s["dtype"]), f"W error {ew} > {tol(s['dtype'])}"
    return eo, ew


__all__ = ["to_device", "run", "err", "tol", "oracle_heads", "gpu_heads", "check", "workloads", "la", "oracle"]
