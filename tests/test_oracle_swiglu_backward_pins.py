"""Pins of the oracle's SwiGLU backward (gradients through the chunk loop:
the read, the eta-weighted gradient step of the binding loss and the column
normalisation), all against computations the oracle does not make itself:
torch autograd of the chunk loop written here (which differentiates through
the inner gradient by double backward), central differences of the oracle's
own forward loop, and mutants."""
import numpy as np
import pytest
import torch

from oracle import ttt_oracle as TO

F = torch.nn.functional


def rand_case(B=1, H=2, T=9, d=4, dh=6, seed=0):
    rng = np.random.default_rng(seed)
    Q, K, V = (rng.standard_normal((B, H, T, d)) for _ in range(3))
    eta = 0.3 * rng.standard_normal((B, H, T))
    W = tuple(0.5 * rng.standard_normal(shp) for shp in ((B, H, d, dh), (B, H, d, dh), (B, H, dh, d)))
    dO = rng.standard_normal((B, H, T, d))
    dW = tuple(rng.standard_normal(w.shape) for w in W)
    return Q, K, V, eta, W, dO, dW


def torch_loop(Q, K, V, eta, W, chunk, read_first, normalize, update_w1w3):
    """The chunk loop in torch: every chunk reads f_W, takes the gradient of sum eta (-<f_W(k), v>) by
    autograd (kept in the graph), steps and normalises."""
    W1, W3, W2 = W
    T = Q.shape[2]
    outs = []
    f = lambda X, a, b, c: (F.silu(X @ a) * (X @ b)) @ c  # noqa: E731
    for s in range(0, T, chunk):
        e = min(s + chunk, T)
        if read_first:
            outs.append(f(Q[:, :, s:e], W1, W3, W2))
        L = -(eta[:, :, s:e] * (f(K[:, :, s:e], W1, W3, W2) * V[:, :, s:e]).sum(-1)).sum()
        g1, g3, g2 = torch.autograd.grad(L, (W1, W3, W2), create_graph=True)
        if update_w1w3:
            W1, W3 = W1 - g1, W3 - g3
        W2 = W2 - g2
        if normalize:
            nz = lambda M: M / M.norm(dim=-2, keepdim=True).clamp_min(1e-12)  # noqa: E731
            W2 = nz(W2)
            if update_w1w3:
                W1, W3 = nz(W1), nz(W3)
        if not read_first:
            outs.append(f(Q[:, :, s:e], W1, W3, W2))
    return torch.cat(outs, 2), (W1, W3, W2)


def autograd_grads(Q, K, V, eta, W, dO, dW, chunk, read_first=True, normalize=True, update_w1w3=True):
    t = lambda a: torch.tensor(a, requires_grad=True)  # noqa: E731
    Qt, Kt, Vt, et = map(t, (Q, K, V, eta))
    Wt = tuple(map(t, W))
    O, WT = torch_loop(Qt, Kt, Vt, et, Wt, chunk, read_first, normalize, update_w1w3)
    loss = (O * torch.tensor(dO)).sum() + sum((a * torch.tensor(b)).sum() for a, b in zip(WT, dW))
    gr = torch.autograd.grad(loss, (Qt, Kt, Vt, et) + Wt)
    return [x.numpy() for x in gr[:4]], [x.numpy() for x in gr[4:]]


@pytest.mark.parametrize("chunk", [1, 3, 4, 9, 20])
@pytest.mark.parametrize("read_first", [True, False])
def test_backward_matches_autograd_of_the_chunk_loop(chunk, read_first):
    Q, K, V, eta, W, dO, dW = rand_case(seed=chunk + 10 * read_first)
    dq, dk, dv, de, G = TO.large_chunk_swiglu_backward(Q, K, V, eta, *W, dO, dW, chunk, read_first=read_first)
    (rq, rk, rv, re), rG = autograd_grads(Q, K, V, eta, W, dO, dW, chunk, read_first)
    for a, b in zip((dq, dk, dv, de) + tuple(G), (rq, rk, rv, re) + tuple(rG)):
        assert np.allclose(a, b, rtol=1e-9, atol=1e-10), np.abs(a - b).max()


@pytest.mark.parametrize("chunk", [1, 4, 9])
def test_backward_last_layer_only_matches_autograd(chunk):
    # W1, W3 fixed, no normalisation: gradients still reach them through the hidden features
    Q, K, V, eta, W, dO, dW = rand_case(seed=30 + chunk)
    res = TO.large_chunk_swiglu_backward(Q, K, V, eta, *W, dO, dW, chunk, normalize=False, update_w1w3=False)
    ref, rG = autograd_grads(Q, K, V, eta, W, dO, dW, chunk, True, False, False)
    for a, b in zip(res[:4] + res[4], ref + rG):
        assert np.allclose(a, b, rtol=1e-9, atol=1e-10)


def test_backward_central_differences_of_the_forward_loop():
    # independent of torch: perturb single entries and difference the oracle's own forward loss
    Q, K, V, eta, W, dO, dW = rand_case(T=7, seed=41)
    chunk = 3
    dq, dk, dv, de, G = TO.large_chunk_swiglu_backward(Q, K, V, eta, *W, dO, dW, chunk)

    def loss(Q_, K_, V_, e_, W_):
        O, WT = TO.large_chunk_swiglu(Q_, K_, V_, e_, *W_, chunk)
        return np.sum(O * dO) + sum(np.sum(a * b) for a, b in zip(WT, dW))

    h = 1e-6
    rng = np.random.default_rng(0)
    for name, arr, grad in (("Q", Q, dq), ("K", K, dk), ("V", V, dv), ("eta", eta, de), ("W1", W[0], G[0]),
                            ("W3", W[1], G[1]), ("W2", W[2], G[2])):
        for _ in range(3):
            idx = tuple(rng.integers(0, n) for n in arr.shape)
            args = {"Q": Q, "K": K, "V": V, "eta": eta}
            Wl = list(W)

            def at(delta):
                a2 = arr.copy()
                a2[idx] += delta
                if name.startswith("W"):
                    Wx = [a2 if k == {"W1": 0, "W3": 1, "W2": 2}[name] else Wl[k] for k in range(3)]
                    return loss(Q, K, V, eta, Wx)
                kw = dict(args)
                kw[name] = a2
                return loss(kw["Q"], kw["K"], kw["V"], kw["eta"], Wl)

            fd = (at(h) - at(-h)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-5 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def test_step_vjp_is_the_double_backward():
    # <D, S(W)> differentiated by torch twice equals the hand-derived product
    Q, K, V, eta, W, dO, dW = rand_case(T=6, seed=42)
    rng = np.random.default_rng(5)
    D = tuple(rng.standard_normal(w.shape) for w in W)
    dk, dv, de, gW = TO.swiglu_step_vjp(K, V, eta, *W, *D)
    t = lambda a: torch.tensor(a, requires_grad=True)  # noqa: E731
    Kt, Vt, et = map(t, (K, V, eta))
    Wt = tuple(map(t, W))
    f = (F.silu(Kt @ Wt[0]) * (Kt @ Wt[1])) @ Wt[2]
    L = (et * (f * Vt).sum(-1)).sum()                    # S = grad of +sum eta <f, v>
    S = torch.autograd.grad(L, Wt, create_graph=True)
    phi = sum((s * torch.tensor(d)).sum() for s, d in zip(S, D))
    ref = torch.autograd.grad(phi, (Kt, Vt, et) + Wt)
    for a, b in zip((dk, dv, de) + tuple(gW), ref):
        assert np.allclose(a, b.numpy(), rtol=1e-10, atol=1e-11)


def test_silu_second_derivative():
    a = torch.linspace(-8, 8, 161, dtype=torch.float64, requires_grad=True)
    (g,) = torch.autograd.grad(F.silu(a).sum(), a, create_graph=True)
    (g2,) = torch.autograd.grad(g.sum(), a)
    assert np.allclose(TO.silu_second(a.detach().numpy()), g2.numpy(), atol=1e-13)
    x = np.linspace(-6, 6, 25)
    fd = (TO.silu_prime(x + 1e-6) - TO.silu_prime(x - 1e-6)) / 2e-6
    assert np.allclose(TO.silu_second(x), fd, atol=1e-8)


def test_zero_cotangents_give_zero_gradients():
    Q, K, V, eta, W, dO, dW = rand_case(seed=43)
    res = TO.large_chunk_swiglu_backward(Q, K, V, eta, *W, np.zeros_like(dO), tuple(np.zeros_like(w) for w in W), 3)
    assert all(np.all(x == 0) for x in res[:4]) and all(np.all(x == 0) for x in res[4])


# ---------------------------------------------------------------------------
# Mutants of the step's vector-Jacobian product: each must fail the autograd pin
# ---------------------------------------------------------------------------

def _vjp_no_second_derivative(K, V, eta, W1, W3, W2, D1, D3, D2):
    orig = TO.silu_second
    TO.silu_second = lambda a: np.zeros_like(a)
    try:
        return _real_vjp(K, V, eta, W1, W3, W2, D1, D3, D2)
    finally:
        TO.silu_second = orig


def _vjp_weights_only_identity(K, V, eta, W1, W3, W2, D1, D3, D2):
    dk, dv, de, gW = _real_vjp(K, V, eta, W1, W3, W2, D1, D3, D2)
    return dk, dv, de, tuple(np.zeros_like(x) for x in gW)


def _vjp_no_tangent_of_w2(K, V, eta, W1, W3, W2, D1, D3, D2):
    return _real_vjp(K, V, eta, W1, W3, W2, D1, D3, np.zeros_like(D2))


def _vjp_eta_missing_in_dv(K, V, eta, W1, W3, W2, D1, D3, D2):
    dk, dv, de, gW = _real_vjp(K, V, eta, W1, W3, W2, D1, D3, D2)
    return dk, dv / np.where(eta[..., None] == 0, 1, eta[..., None]), de, gW


_real_vjp = TO.swiglu_step_vjp


@pytest.mark.parametrize("mutant", [_vjp_no_second_derivative, _vjp_weights_only_identity, _vjp_no_tangent_of_w2,
                                    _vjp_eta_missing_in_dv])
def test_mutants_of_the_step_product_are_caught(mutant, monkeypatch):
    Q, K, V, eta, W, dO, dW = rand_case(seed=44)
    (rq, rk, rv, re), rG = autograd_grads(Q, K, V, eta, W, dO, dW, 3)
    monkeypatch.setattr(TO, "swiglu_step_vjp", mutant)
    dq, dk, dv, de, G = TO.large_chunk_swiglu_backward(Q, K, V, eta, *W, dO, dW, 3)
    same = all(np.allclose(a, b, rtol=1e-6, atol=1e-8) for a, b in zip((dq, dk, dv, de) + tuple(G),
                                                                          (rq, rk, rv, re) + tuple(rG)))
    assert not same
