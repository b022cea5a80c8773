"""Seeded synthetic inputs for the TTT-layer forward pass.

Shared by the tests, the smoke check and the benchmark; holds none of the
method's arithmetic (no update, read or normalisation of fast weights), only
the input recipe:

* NumPy PCG64 ``default_rng(seed)``; draws in the order Q, K, V, eta, then
  the initial fast weights (W0, or W1, W3, W2 for the SwiGLU memory), all
  float32;
* queries and keys are divided by their per-token L2 norm (a property of the
  workloads' inputs; the operation itself never normalises them);
* eta is ``U(0, s)`` or ``sigmoid(N(0,1)) * s`` per (b, h, t);
* initial weights are zero or ``N(0, std^2)`` drawn once per head and
  broadcast over the batch;
* for bf16 workloads Q, K and V are rounded to bfloat16 (round to nearest,
  ties to even); eta and the weights stay float32.

Every array is returned as float32 holding exactly the values the GPU sees,
so the oracle can up-cast them without counting input quantisation as error.
"""
from __future__ import annotations

import numpy as np

MODES = ("per_token_linear", "large_chunk_linear", "large_chunk_swiglu",
         # the other read orders: a query before its token's step; a chunk's step before its reads
         "per_token_linear_exclusive", "large_chunk_linear_update_first", "large_chunk_swiglu_update_first",
         # SwiGLU with only W2 trained and no normalisation
         "large_chunk_swiglu_last_layer")

# Named workloads.  Shapes follow the configurations the method is measured
# on; T is the sequence length, d the head width, d_h the SwiGLU hidden width.
WORKLOADS = {
    "per_token_fp32_B1H1T256_d64_c64": dict(
        mode="per_token_linear", B=1, H=1, T=256, d_k=64, d_v=64, d_h=0, chunk=64,
        dtype="fp32", eta="uniform", eta_scale=0.1, w0="zero", w0_std=0.0),
    "per_token_bf16_B4H16T4096_d128_c64": dict(
        mode="per_token_linear", B=4, H=16, T=4096, d_k=128, d_v=128, d_h=0, chunk=64,
        dtype="bf16", eta="sigmoid", eta_scale=0.1, w0="normal", w0_std=0.02),
    # O in float32: rounding even the exact outputs of these 32 heads to bf16 would exceed 2% of their RMS
    "per_token_bf16_B1H32T32768_d128_c128": dict(
        mode="per_token_linear", B=1, H=32, T=32768, d_k=128, d_v=128, d_h=0, chunk=128,
        dtype="bf16", eta="sigmoid", eta_scale=0.1, w0="normal", w0_std=0.02, o_dtype="fp32"),
    "large_chunk_linear_bf16_B1H12T196608_d64_c4096": dict(
        mode="large_chunk_linear", B=1, H=12, T=196608, d_k=64, d_v=64, d_h=0, chunk=4096,
        dtype="bf16", eta="uniform", eta_scale=0.05, w0="normal", w0_std=0.02),
    "large_chunk_swiglu_bf16_B2H8T32768_d128_dh256_c2048": dict(
        mode="large_chunk_swiglu", B=2, H=8, T=32768, d_k=128, d_v=128, d_h=256, chunk=2048,
        dtype="bf16", eta="uniform", eta_scale=0.02, w0="normal", w0_std=0.02),
}

# The workload the headline throughput is quoted on: the largest of the per-token mode.
HEADLINE = "per_token_bf16_B1H32T32768_d128_c128"


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even) and
    return them as float32 (finite inputs only: for those the sum below
    stays under 2^32)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def spec(name: str, **overrides) -> dict:
    """A copy of a named workload's parameters with overrides applied.
    ``o_dtype`` is the element type of the outputs O (the input dtype
    unless the workload names another)."""
    s = dict(WORKLOADS[name])
    s.setdefault("o_dtype", s["dtype"])
    s.update(overrides)
    return s


def make_spec(mode, B, H, T, d_k, d_v=None, d_h=0, chunk=64, dtype="bf16",
              eta="uniform", eta_scale=0.1, w0="normal", w0_std=0.02, o_dtype=None) -> dict:
    """Build a workload parameter dict for an arbitrary shape."""
    assert mode in MODES
    return dict(mode=mode, B=B, H=H, T=T, d_k=d_k, d_v=d_k if d_v is None else d_v,
                d_h=d_h, chunk=chunk, dtype=dtype, eta=eta, eta_scale=eta_scale,
                w0=w0, w0_std=w0_std, o_dtype=dtype if o_dtype is None else o_dtype)


def generate(s: dict, seed: int = 0) -> dict:
    """Draw one batch of inputs for workload parameters ``s``.

    Returns float32 arrays ``Q, K, V, eta, W0``; for the SwiGLU memory W0 is
    the packed per-head state ``[B,H, d*d_h (W1) + d*d_h (W3) + d_h*d (W2)]``
    and ``W1, W3, W2`` are also returned unpacked."""
    B, H, T, dk, dv, dh = s["B"], s["H"], s["T"], s["d_k"], s["d_v"], s["d_h"]
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, H, T, dk), dtype=np.float32)
    K = rng.standard_normal((B, H, T, dk), dtype=np.float32)
    V = rng.standard_normal((B, H, T, dv), dtype=np.float32)
    if s["eta"] == "uniform":
        eta = rng.uniform(0.0, s["eta_scale"], size=(B, H, T)).astype(np.float32)
    elif s["eta"] == "sigmoid":
        z = rng.standard_normal((B, H, T))
        eta = (s["eta_scale"] / (1.0 + np.exp(-z))).astype(np.float32)
    elif s["eta"] == "normal":
        eta = (s["eta_scale"] * rng.standard_normal((B, H, T))).astype(np.float32)
    else:
        raise ValueError(s["eta"])
    for X in (Q, K):
        n = np.sqrt(np.sum(X.astype(np.float64) ** 2, axis=-1, keepdims=True))
        X /= np.maximum(n, 1e-30).astype(np.float32)
    if s["dtype"] == "bf16":
        Q, K, V = bf16_round(Q), bf16_round(K), bf16_round(V)
    out = dict(Q=Q, K=K, V=V, eta=eta)

    def draw(shape):
        if s["w0"] == "zero":
            w = np.zeros((H,) + shape, dtype=np.float32)
        else:
            w = (s["w0_std"] * rng.standard_normal((H,) + shape)).astype(np.float32)
        return np.ascontiguousarray(np.broadcast_to(w[None], (B, H) + shape))

    if s["mode"].startswith("large_chunk_swiglu"):
        assert dk == dv and dh > 0
        W1, W3, W2 = draw((dk, dh)), draw((dk, dh)), draw((dh, dk))
        out.update(W1=W1, W3=W3, W2=W2, W0=np.concatenate(
            [W1.reshape(B, H, -1), W3.reshape(B, H, -1), W2.reshape(B, H, -1)], axis=-1))
    else:
        out["W0"] = draw((dk, dv))
    return out


def generate_grads(s: dict, seed: int = 0) -> dict:
    """Upstream gradients for a backward pass over the inputs of ``s``:
    ``dO`` ``[B,H,T,d_v]`` ~ N(0, 1) (bf16-representable for bf16 inputs)
    and ``dW`` ~ N(0, 1) in the state's shape (packed W1 | W3 | W2 for the
    SwiGLU memory), from a generator stream of their own (the forward
    inputs do not change)."""
    B, H, T, dv = s["B"], s["H"], s["T"], s["d_v"]
    rng = np.random.default_rng([seed, 1])
    dO = rng.standard_normal((B, H, T, dv), dtype=np.float32)
    if s["dtype"] == "bf16":
        dO = bf16_round(dO)
    dW = rng.standard_normal(state_shape(s), dtype=np.float32)
    return dict(dO=dO, dW=dW)


def state_shape(s: dict) -> tuple:
    """Shape of the fast-weight state buffer (W0 and W_out) for ``s``."""
    if s["mode"].startswith("large_chunk_swiglu"):
        return (s["B"], s["H"], 3 * s["d_k"] * s["d_h"])
    return (s["B"], s["H"], s["d_k"], s["d_v"])
