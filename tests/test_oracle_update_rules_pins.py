"""Pins of the oracle's other update rules for the SwiGLU memory (LaCT review,
non-linear memory section: gradient descent, momentum and Muon, whose
Newton-Schulz iterations transform the matrix gradients, with the L2
normalisation after the update).

Each pin checks the oracle against something it does not compute itself: the
singular-value form of the Newton-Schulz map (from numpy's SVD and a scalar
polynomial written out here), chunk steps rebuilt by hand from torch autograd
gradients, and the plain update rule the variants reduce to.
"""
import numpy as np
import pytest
import torch

from oracle import ttt_oracle as TO

A_, B_, C_ = 3.4445, -4.7750, 2.0315      # Muon's published quintic


def rand_swiglu(B=1, H=2, T=10, d=4, dh=6, seed=0, eta_scale=0.3):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, H, T, d))
    K = rng.standard_normal((B, H, T, d))
    V = rng.standard_normal((B, H, T, d))
    eta = eta_scale * rng.standard_normal((B, H, T))
    W1 = 0.5 * rng.standard_normal((B, H, d, dh))
    W3 = 0.5 * rng.standard_normal((B, H, d, dh))
    W2 = 0.5 * rng.standard_normal((B, H, dh, d))
    return Q, K, V, eta, W1, W3, W2


def quintic5(s):
    """The scalar map the iteration applies to every singular value, five times."""
    for _ in range(5):
        s = A_ * s + B_ * s ** 3 + C_ * s ** 5
    return s


def ns_by_svd(G):
    """Newton-Schulz result written through the SVD of G: U diag(p(s / (||G||_F + 1e-7))) V^T."""
    U, s, Vt = np.linalg.svd(G, full_matrices=False)
    f = np.sqrt(np.sum(G * G)) + 1e-7
    return (U * np.array([quintic5(x / f) for x in s])) @ Vt


@pytest.mark.parametrize("shape,rank", [((6, 10), None), ((10, 6), None), ((8, 8), None), ((6, 10), 2),
                                        ((1, 5), None)])
def test_newton_schulz_is_the_quintic_on_singular_values(shape, rank):
    rng = np.random.default_rng(sum(shape) + (rank or 0))
    G = rng.standard_normal(shape)
    if rank:
        G = rng.standard_normal((shape[0], rank)) @ rng.standard_normal((rank, shape[1]))
    assert np.allclose(TO.newton_schulz5(G), ns_by_svd(G), atol=1e-11)


def test_newton_schulz_band_on_well_conditioned_inputs():
    # singular values spread over a factor of 3 all land near 1 (the quintic's band)
    rng = np.random.default_rng(3)
    Ua, _ = np.linalg.qr(rng.standard_normal((16, 16)))
    Vb, _ = np.linalg.qr(rng.standard_normal((32, 16)))
    G = (Ua * np.linspace(1.0, 3.0, 16)) @ Vb.T
    s = np.linalg.svd(TO.newton_schulz5(G), compute_uv=False)
    assert s.min() > 0.6 and s.max() < 1.25, s


def test_newton_schulz_batched_and_transposed():
    rng = np.random.default_rng(4)
    G = rng.standard_normal((2, 3, 5, 7))
    X = TO.newton_schulz5(G)
    for i in range(2):
        for j in range(3):
            assert np.allclose(X[i, j], ns_by_svd(G[i, j]), atol=1e-11)
    assert np.allclose(TO.newton_schulz5(np.swapaxes(G, -1, -2)), np.swapaxes(X, -1, -2), atol=1e-12)


def torch_grads(K, V, eta, W1, W3, W2):
    """Gradients of sum_i eta_i (-<f_W(k_i), v_i>) by torch autograd."""
    ws = [torch.tensor(w, requires_grad=True) for w in (W1, W3, W2)]
    Kt, Vt, et = map(torch.tensor, (K, V, eta))
    f = (torch.nn.functional.silu(Kt @ ws[0]) * (Kt @ ws[1])) @ ws[2]
    (-(et * (f * Vt).sum(-1)).sum()).backward()
    return [w.grad.numpy() for w in ws]


def torch_mlp(X, W1, W3, W2):
    t = torch.tensor
    return ((torch.nn.functional.silu(t(X) @ t(W1)) * (t(X) @ t(W3))) @ t(W2)).numpy()


def colnorm(W):
    return W / np.linalg.norm(W, axis=-2, keepdims=True)


def by_hand(Q, K, V, eta, W, chunk, beta=None, muon=None):
    """The chunk loop rebuilt from torch gradients: momentum buffers, then the (SVD-form) Newton-Schulz map,
    then the normalisation; read before the update."""
    W = [w.copy() for w in W]
    M = [np.zeros_like(w) for w in W]
    T = Q.shape[2]
    O = np.zeros(Q.shape)
    for s in range(0, T, chunk):
        e = min(s + chunk, T)
        O[:, :, s:e] = torch_mlp(Q[:, :, s:e], *W)
        g = torch_grads(K[:, :, s:e], V[:, :, s:e], eta[:, :, s:e], *W)
        step = [-x for x in g]
        if beta is not None:
            M = [beta * m + st for m, st in zip(M, step)]
            step = list(M)
        if muon is not None:
            step = [muon * np.stack([np.stack([ns_by_svd(x[b, h]) for h in range(x.shape[1])])
                                     for b in range(x.shape[0])]) for x in step]
        W = [colnorm(w + st) for w, st in zip(W, step)]
    return O, W, M


def test_momentum_zero_is_plain_descent():
    Q, K, V, eta, W1, W3, W2 = rand_swiglu(seed=20)
    O, W = TO.large_chunk_swiglu(Q, K, V, eta, W1, W3, W2, 4)
    Om, Wm, M = TO.large_chunk_swiglu(Q, K, V, eta, W1, W3, W2, 4, momentum=0.0)
    assert np.array_equal(O, Om) and all(np.array_equal(a, b) for a, b in zip(W, Wm))


@pytest.mark.parametrize("beta,muon", [(0.9, None), (None, 0.3), (0.8, 0.5)])
def test_update_rules_three_chunks_by_hand(beta, muon):
    Q, K, V, eta, W1, W3, W2 = rand_swiglu(T=11, seed=21)
    kw = {}
    if beta is not None:
        kw["momentum"] = beta
    if muon is not None:
        kw["muon_scale"] = muon
    res = TO.large_chunk_swiglu(Q, K, V, eta, W1, W3, W2, 4, **kw)
    Oh, Wh, Mh = by_hand(Q, K, V, eta, [W1, W3, W2], 4, beta, muon)
    assert np.allclose(res[0], Oh, atol=1e-10)
    assert all(np.allclose(a, b, atol=1e-10) for a, b in zip(res[1], Wh))
    if beta is not None:
        assert all(np.allclose(a, b, atol=1e-10) for a, b in zip(res[2], Mh))


def test_momentum_resume_with_buffers():
    Q, K, V, eta, W1, W3, W2 = rand_swiglu(T=12, seed=22)
    O, W, M = TO.large_chunk_swiglu(Q, K, V, eta, W1, W3, W2, 4, momentum=0.7, muon_scale=0.2)
    sl = lambda a, s: a[:, :, s]  # noqa: E731
    a, b = slice(0, 8), slice(8, 12)
    Oa, Wa, Ma = TO.large_chunk_swiglu(sl(Q, a), sl(K, a), sl(V, a), sl(eta, a), W1, W3, W2, 4, momentum=0.7,
                                       muon_scale=0.2)
    Ob, Wb, Mb = TO.large_chunk_swiglu(sl(Q, b), sl(K, b), sl(V, b), sl(eta, b), *Wa, 4, momentum=0.7, M0=Ma,
                                       muon_scale=0.2)
    assert np.allclose(np.concatenate([Oa, Ob], 2), O, atol=1e-12)
    assert all(np.allclose(x, y, atol=1e-12) for x, y in zip(Wb, W))
    assert all(np.allclose(x, y, atol=1e-12) for x, y in zip(Mb, M))


def test_muon_step_has_unit_band_before_normalisation():
    # with the normalisation off, a single Muon step of scale s moves each matrix by s times an
    # (approximately) orthogonal matrix: its singular values sit in the quintic's band
    Q, K, V, eta, W1, W3, W2 = rand_swiglu(T=40, d=6, dh=12, seed=23)
    _, (N1, N3, N2) = TO.large_chunk_swiglu(Q, K, V, eta, W1, W3, W2, 40, normalize=False, muon_scale=1.0)
    for new, old in ((N1, W1), (N3, W3), (N2, W2)):
        s = np.linalg.svd((new - old)[0, 0], compute_uv=False)
        assert s.max() < 1.25 and s.min() > 0.3, s


# ---------------------------------------------------------------------------
# Mutants: plausible mistakes in the iteration must fail the singular-value pin
# ---------------------------------------------------------------------------

def _ns_wrong_sign(G):
    a, b, c = A_, -B_, C_
    X = G / (np.linalg.norm(G) + 1e-7)
    for _ in range(5):
        A = X @ X.T
        X = a * X + (b * A + c * A @ A) @ X
    return X


def _ns_spectral_norm(G):
    X = G / np.linalg.norm(G, 2)
    for _ in range(5):
        A = X @ X.T
        X = A_ * X + (B_ * A + C_ * A @ A) @ X
    return X


def _ns_unnormalised(G):
    X = G.copy()
    for _ in range(5):
        A = X @ X.T
        X = A_ * X + (B_ * A + C_ * A @ A) @ X
    return X


def _ns_four_steps(G):
    X = G / (np.linalg.norm(G) + 1e-7)
    for _ in range(4):
        A = X @ X.T
        X = A_ * X + (B_ * A + C_ * A @ A) @ X
    return X


@pytest.mark.parametrize("mutant", [_ns_wrong_sign, _ns_spectral_norm, _ns_unnormalised, _ns_four_steps])
def test_newton_schulz_mutants_are_caught(mutant):
    rng = np.random.default_rng(9)
    caught = False
    for shape in ((6, 10), (10, 6)):
        G = 0.3 * rng.standard_normal(shape)
        with np.errstate(all="ignore"):
            X = mutant(G)
        if not np.all(np.isfinite(X)) or not np.allclose(X, ns_by_svd(G), atol=1e-6):
            caught = True
    assert caught
