"""Pins of the oracle's per-token and large-chunk linear backward (CPU only).

The hand-derived reverse loop is checked against things it does not share
code with: torch autograd of the per-token closed form written here with
cumulative sums, central finite differences of the oracle's own forward
loop, the closed form of dW0, and the zero-rate special case.  Shapes use
d_k != d_v so that a transposed operand cannot pass.  Mutation tests plant
typical mistakes in copies of the backward and check that a pin catches each.
"""
import numpy as np
import pytest
import torch

from oracle import ttt_oracle as TO


def case(B=2, H=2, T=11, dk=5, dv=3, seed=0, eta_scale=0.4):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, H, T, dk))
    K = rng.standard_normal((B, H, T, dk))
    V = rng.standard_normal((B, H, T, dv))
    eta = eta_scale * rng.standard_normal((B, H, T))
    W0 = 0.3 * rng.standard_normal((B, H, dk, dv))
    dO = rng.standard_normal((B, H, T, dv))
    dW = rng.standard_normal((B, H, dk, dv))
    return Q, K, V, eta, W0, dO, dW


def autograd_grads(Q, K, V, eta, W0, dO, dW, inclusive):
    """Gradients of sum(O * dO) + sum(W_T * dW) through the closed form
    S_t = W0 + sum_{i<=t} eta_i k_i^T v_i, o_t = q_t S_t (S_{t-1} when not inclusive)."""
    xs = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (Q, K, V, eta, W0)]
    q, k, v, e, w0 = xs
    outer = (e[..., None, None] * k[..., :, None]) * v[..., None, :]          # [B,H,T,dk,dv]
    S = w0[:, :, None] + torch.cumsum(outer, dim=2)                          # S_t, t = 0..T-1
    if not inclusive:
        S = torch.cat([w0[:, :, None], S[:, :, :-1]], dim=2)                 # S_{t-1}
    O = torch.matmul(q[..., None, :], S)[..., 0, :]
    WT = w0 + outer.sum(dim=2)
    loss = (O * torch.from_numpy(dO)).sum() + (WT * torch.from_numpy(dW)).sum()
    loss.backward()
    return [x.grad.numpy() for x in xs]


def check_autograd(bwd=TO.per_token_linear_backward, inclusive=True, seed=0, **kw):
    Q, K, V, eta, W0, dO, dW = case(seed=seed, **kw)
    got = bwd(Q, K, V, eta, W0, dO, dW, inclusive=inclusive)
    ref = autograd_grads(Q, K, V, eta, W0, dO, dW, inclusive)
    return all(np.allclose(g, r, rtol=1e-10, atol=1e-10) for g, r in zip(got, ref))


def check_finite_differences(bwd=TO.per_token_linear_backward, inclusive=True, seed=1):
    """<grad_X, delta> against a central difference of the forward loop's loss, for every input."""
    args = list(case(B=1, H=2, T=7, dk=4, dv=3, seed=seed))
    dO, dW = args[5], args[6]
    grads = bwd(*args, inclusive=inclusive)
    rng = np.random.default_rng(seed + 100)

    def loss(a):
        O, WT = TO.per_token_linear(*a[:5], inclusive=inclusive)
        return float(np.sum(O * dO) + np.sum(WT * dW))

    h = 1e-6
    ok = True
    for i in range(5):
        delta = rng.standard_normal(args[i].shape)
        ap, am = list(args), list(args)
        ap[i] = args[i] + h * delta
        am[i] = args[i] - h * delta
        fd = (loss(ap) - loss(am)) / (2 * h)
        an = float(np.sum(grads[i] * delta))
        ok &= abs(fd - an) <= 1e-6 * max(1.0, abs(an))
    return ok


@pytest.mark.parametrize("inclusive", [True, False])
@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_autograd_of_the_closed_form(inclusive, seed):
    assert check_autograd(inclusive=inclusive, seed=seed)


@pytest.mark.parametrize("inclusive", [True, False])
def test_backward_matches_autograd_single_token_and_square(inclusive):
    assert check_autograd(inclusive=inclusive, T=1)
    assert check_autograd(inclusive=inclusive, dk=4, dv=4, T=6)


@pytest.mark.parametrize("inclusive", [True, False])
def test_backward_matches_finite_differences_of_the_forward_loop(inclusive):
    assert check_finite_differences(inclusive=inclusive)


@pytest.mark.parametrize("inclusive", [True, False])
def test_dW0_closed_form(inclusive):
    # W0 enters every read and the final memory once: dW0 = dW + sum_t q_t^T dO_t
    Q, K, V, eta, W0, dO, dW = case(seed=3)
    dW0 = TO.per_token_linear_backward(Q, K, V, eta, W0, dO, dW, inclusive=inclusive)[4]
    assert np.allclose(dW0, dW + np.swapaxes(Q, -1, -2) @ dO, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("inclusive", [True, False])
def test_zero_rate(inclusive):
    # eta = 0: the memory stays W0, so dQ = dO W0^T and no gradient reaches K or V; deta_t is
    # k_t G_t v_t^T with G_t = dW + sum over the reads that come after step t
    Q, K, V, eta, W0, dO, dW = case(seed=4)
    eta = np.zeros_like(eta)
    dQ, dK, dV, deta, _ = TO.per_token_linear_backward(Q, K, V, eta, W0, dO, dW, inclusive=inclusive)
    assert np.allclose(dQ, dO @ np.swapaxes(W0, -1, -2), rtol=1e-12, atol=1e-12)
    assert not dK.any() and not dV.any()
    T = Q.shape[2]
    for t in range(T):
        lo = t if inclusive else t + 1
        G = dW + np.swapaxes(Q[:, :, lo:], -1, -2) @ dO[:, :, lo:]
        ref = (K[:, :, t, None, :] @ G @ V[:, :, t, :, None])[..., 0, 0]
        assert np.allclose(deta[:, :, t], ref, rtol=1e-12, atol=1e-12)


def test_backward_dispatch():
    Q, K, V, eta, W0, dO, dW = case(seed=5)
    for mode, inc in (("per_token_linear", True), ("per_token_linear_exclusive", False)):
        a = TO.backward(Q, K, V, eta, W0, dO, dW, 64, mode)
        b = TO.per_token_linear_backward(Q, K, V, eta, W0, dO, dW, inclusive=inc)
        assert all(np.array_equal(x, y) for x, y in zip(a, b))
    for mode, rf in (("large_chunk_linear", True), ("large_chunk_linear_update_first", False)):
        a = TO.backward(Q, K, V, eta, W0, dO, dW, 4, mode)
        b = TO.large_chunk_linear_backward(Q, K, V, eta, W0, dO, dW, 4, read_first=rf)
        assert all(np.array_equal(x, y) for x, y in zip(a, b))
    with pytest.raises(ValueError):
        TO.backward(Q, K, V, eta, W0, dO, dW, 64, "no_such_mode")
    # SwiGLU: packed states in and out, the three modes' flags
    rng = np.random.default_rng(6)
    B, H, T, d, dh = 1, 2, 7, 4, 6
    Qs, Ks, Vs, dOs = (rng.standard_normal((B, H, T, d)) for _ in range(4))
    es = 0.3 * rng.standard_normal((B, H, T))
    Ws = [0.5 * rng.standard_normal(shp) for shp in ((B, H, d, dh), (B, H, d, dh), (B, H, dh, d))]
    dWs = [rng.standard_normal(w.shape) for w in Ws]
    for mode, kw in (("large_chunk_swiglu", {}), ("large_chunk_swiglu_update_first", dict(read_first=False)),
                     ("large_chunk_swiglu_last_layer", dict(normalize=False, update_w1w3=False))):
        a = TO.backward(Qs, Ks, Vs, es, TO.swiglu_pack(*Ws), dOs, TO.swiglu_pack(*dWs), 3, mode, d_h=dh)
        b = TO.large_chunk_swiglu_backward(Qs, Ks, Vs, es, *Ws, dOs, dWs, 3, **kw)
        assert all(np.array_equal(x, y) for x, y in zip(a[:4], b[:4]))
        assert np.array_equal(a[4], TO.swiglu_pack(*b[4]))


# ---------------------------------------------------------------------------
# Mutation tests
# ---------------------------------------------------------------------------

def _mutant(kind):
    def bwd(Q, K, V, eta, W0, dO, dW, inclusive=True):
        dQ, dK, dV, deta, dW0 = TO.per_token_linear_backward(Q, K, V, eta, W0, dO, dW, inclusive=inclusive)
        if kind == "dk_without_eta":
            dK = np.where(np.abs(eta[..., None]) > 0, dK / eta[..., None], 0.0)
        elif kind == "dv_sign":
            dV = -dV
        elif kind == "dropped_final_state_gradient":
            dQ, dK, dV, deta, dW0 = TO.per_token_linear_backward(Q, K, V, eta, W0, dO, 0 * dW, inclusive=inclusive)
        elif kind == "other_read_order":
            dQ, dK, dV, deta, dW0 = TO.per_token_linear_backward(Q, K, V, eta, W0, dO, dW, inclusive=not inclusive)
        elif kind == "deta_sign":
            deta = -deta
        elif kind == "dq_from_initial_memory":
            dQ = dO @ np.swapaxes(W0, -1, -2)
        return dQ, dK, dV, deta, dW0
    return bwd


@pytest.mark.parametrize("kind", ["dk_without_eta", "dv_sign", "dropped_final_state_gradient", "other_read_order",
                                  "deta_sign", "dq_from_initial_memory"])
def test_backward_mutants_are_caught(kind):
    m = _mutant(kind)
    assert not (check_autograd(bwd=m, inclusive=True) and check_finite_differences(bwd=m, inclusive=True))



# ---------------------------------------------------------------------------
# Large-chunk linear backward
# ---------------------------------------------------------------------------

def lact_autograd(Q, K, V, eta, W0, dO, dW, chunk, read_first):
    """Gradients of sum(O * dO) + sum(W_T * dW) through the chunk loop written with torch ops
    (column norms clamped at 1e-12), by autograd."""
    xs = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (Q, K, V, eta, W0)]
    q, k, v, e, W = xs
    T = q.shape[2]
    outs = []
    for s in range(0, T, chunk):
        sl = slice(s, min(s + chunk, T))
        if read_first:
            outs.append(torch.matmul(q[:, :, sl], W))
        P = W + torch.matmul(k[:, :, sl].transpose(-1, -2), e[:, :, sl, None] * v[:, :, sl])
        W = P / torch.linalg.vector_norm(P, dim=-2, keepdim=True).clamp_min(1e-12)
        if not read_first:
            outs.append(torch.matmul(q[:, :, sl], W))
    O = torch.cat(outs, dim=2)
    loss = (O * torch.from_numpy(dO)).sum() + (W * torch.from_numpy(dW)).sum()
    loss.backward()
    return [x.grad.numpy() for x in xs]


def check_lact_autograd(bwd=TO.large_chunk_linear_backward, read_first=True, chunk=4, seed=0, **kw):
    Q, K, V, eta, W0, dO, dW = case(seed=seed, **kw)
    got = bwd(Q, K, V, eta, W0, dO, dW, chunk, read_first=read_first)
    ref = lact_autograd(Q, K, V, eta, W0, dO, dW, chunk, read_first)
    return all(np.allclose(g, r, rtol=1e-9, atol=1e-9) for g, r in zip(got, ref))


@pytest.mark.parametrize("read_first", [True, False])
@pytest.mark.parametrize("chunk", [1, 3, 4, 11, 20])
def test_lact_backward_matches_autograd(read_first, chunk):
    assert check_lact_autograd(read_first=read_first, chunk=chunk)
    assert check_lact_autograd(read_first=read_first, chunk=chunk, seed=1, dk=4, dv=4)


@pytest.mark.parametrize("read_first", [True, False])
def test_lact_backward_matches_finite_differences(read_first):
    args = list(case(B=1, H=2, T=9, dk=4, dv=3, seed=2))
    dO, dW = args[5], args[6]
    grads = TO.large_chunk_linear_backward(*args, 4, read_first=read_first)
    rng = np.random.default_rng(7)

    def loss(a):
        O, WT = TO.large_chunk_linear(*a[:5], 4, read_first=read_first)
        return float(np.sum(O * dO) + np.sum(WT * dW))

    h = 1e-6
    for i in range(5):
        delta = rng.standard_normal(args[i].shape)
        ap, am = list(args), list(args)
        ap[i] = args[i] + h * delta
        am[i] = args[i] - h * delta
        fd = (loss(ap) - loss(am)) / (2 * h)
        an = float(np.sum(grads[i] * delta))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an))


def test_lact_backward_zero_rate_and_normalised_start():
    # eta = 0 with unit-column W0: the memory never changes (a fixed point of the normalisation), so
    # dQ = dO W0^T in both orders and K and V get nothing.  Every gradient that passes through a
    # normalisation of a unit column is projected onto that column's tangent space: dW0 is orthogonal
    # to W0 column by column when the first chunk updates before it reads, and so is dW0 - Q_0^T dO_0
    # (the first chunk's read of W0 itself) when it reads first.
    Q, K, V, eta, W0, dO, dW = case(seed=6)
    W0 = W0 / np.linalg.norm(W0, axis=-2, keepdims=True)
    eta = np.zeros_like(eta)
    for rf in (True, False):
        dQ, dK, dV, deta, dW0 = TO.large_chunk_linear_backward(Q, K, V, eta, W0, dO, dW, 4, read_first=rf)
        assert np.allclose(dQ, dO @ np.swapaxes(W0, -1, -2), rtol=1e-12, atol=1e-12)
        assert not dK.any() and not dV.any()
        tangent = dW0 - np.swapaxes(Q[:, :, :4], -1, -2) @ dO[:, :, :4] if rf else dW0
        assert np.allclose(np.sum(tangent * W0, axis=-2), 0.0, atol=1e-9)


@pytest.mark.parametrize("kind", ["no_projection", "dq_from_new_memory", "g_reset"])
def test_lact_backward_mutants_are_caught(kind):
    def bwd(Q, K, V, eta, W0, dO, dW, chunk, read_first=True):
        if kind == "dq_from_new_memory":
            return TO.large_chunk_linear_backward(Q, K, V, eta, W0, dO, dW, chunk, read_first=not read_first)
        g = list(TO.large_chunk_linear_backward(Q, K, V, eta, W0, dO, dW, chunk, read_first=read_first))
        if kind == "no_projection":
            # normalisation treated as a constant scale: drop the tangent projection
            g[1] = g[1] * 1.01
        elif kind == "g_reset":
            g[4] = dW + np.swapaxes(Q, -1, -2) @ dO
        return tuple(g)
    assert not check_lact_autograd(bwd=bwd, read_first=True)
