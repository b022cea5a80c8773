"""Pins for the fp64 oracle (CPU only).

The oracle is pinned to things other than itself: hand-worked examples
(tests/golden), closed forms (causal linear attention, an MLP forward),
automatic and finite-difference gradients, special cases and invariants.
The mutation tests at the end plant typical mistakes in copies of the oracle
and check that at least one pin catches each of them.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import ttt_oracle as TO
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def rand_case(B=2, H=2, T=13, dk=5, dv=4, seed=0, eta_scale=0.3):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, H, T, dk))
    K = rng.standard_normal((B, H, T, dk))
    V = rng.standard_normal((B, H, T, dv))
    eta = eta_scale * rng.standard_normal((B, H, T))
    W0 = 0.3 * rng.standard_normal((B, H, dk, dv))
    return Q, K, V, eta, W0


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


# ---------------------------------------------------------------------------
# Hand-worked examples
# ---------------------------------------------------------------------------

def _golden():
    with open(GOLDEN) as f:
        g = json.load(f)
    inp = {k: np.array(v, dtype=np.float64) for k, v in g["inputs"].items()}
    add = lambda x: x[None, None]  # noqa: E731  (B = H = 1)
    return g, add(inp["Q"]), add(inp["K"]), add(inp["V"]), add(inp["eta"]), add(inp["W0"])


def check_golden(pt=TO.per_token_linear, lcl=TO.large_chunk_linear):
    g, Q, K, V, eta, W0 = _golden()
    ok = True
    O, W = pt(Q, K, V, eta, W0)
    ok &= np.allclose(O[0, 0], g["per_token_inclusive"]["O"], atol=1e-14)
    ok &= np.allclose(W[0, 0], g["per_token_inclusive"]["W"], atol=1e-14)
    O, W = pt(Q, K, V, eta, W0, inclusive=False)
    ok &= np.allclose(O[0, 0], g["per_token_exclusive"]["O"], atol=1e-14)
    ok &= np.allclose(W[0, 0], g["per_token_exclusive"]["W"], atol=1e-14)
    O, W = lcl(Q, K, V, eta, W0, 2)
    ok &= np.allclose(O[0, 0], g["large_chunk_linear_chunk2"]["O"], atol=1e-13)
    ok &= np.allclose(W[0, 0], g["large_chunk_linear_chunk2"]["W"], atol=1e-13)
    return bool(ok)


def test_golden_hand_examples():
    assert check_golden()


# ---------------------------------------------------------------------------
# P-1: per-token mode equals the causal linear-attention closed form
# ---------------------------------------------------------------------------

def brute_force_linear_attention(Q, K, V, eta, W0, inclusive=True):
    """o_t = q_t W0 + sum_{i<=t (or <t)} (q_t . k_i) eta_i v_i, by plain loops."""
    B, H, T, dk = Q.shape
    dv = V.shape[-1]
    O = np.zeros((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            for t in range(T):
                acc = [sum(Q[b, h, t, a] * W0[b, h, a, j] for a in range(dk)) for j in range(dv)]
                last = t + 1 if inclusive else t
                for i in range(last):
                    s = sum(Q[b, h, t, a] * K[b, h, i, a] for a in range(dk)) * eta[b, h, i]
                    for j in range(dv):
                        acc[j] += s * V[b, h, i, j]
                O[b, h, t] = acc
    return O


def check_closed_form(pt=TO.per_token_linear, seed=0):
    Q, K, V, eta, W0 = rand_case(B=1, H=2, T=9, dk=3, dv=4, seed=seed)
    ok = True
    for inclusive in (True, False):
        O, W = pt(Q, K, V, eta, W0, inclusive=inclusive)
        ref = brute_force_linear_attention(Q, K, V, eta, W0, inclusive)
        ok &= np.allclose(O, ref, atol=1e-12, rtol=0)
        Wref = W0.copy()
        for b in range(W0.shape[0]):
            for h in range(W0.shape[1]):
                for i in range(Q.shape[2]):
                    Wref[b, h] += eta[b, h, i] * np.outer(K[b, h, i], V[b, h, i])
        ok &= np.allclose(W, Wref, atol=1e-12, rtol=0)
    return bool(ok)


def test_p1_closed_form_brute_force():
    assert check_closed_form()


def test_p1_closed_form_matrix_larger():
    # Matrix form O = Q W0 + (tril(Q K^T) * eta_j) V on a mid-sized case.
    Q, K, V, eta, W0 = rand_case(B=2, H=3, T=40, dk=8, dv=6, seed=3)
    O, W = TO.per_token_linear(Q, K, V, eta, W0)
    P = np.tril(np.matmul(Q, np.swapaxes(K, -1, -2))) * eta[:, :, None, :]
    assert np.allclose(O, np.matmul(Q, W0) + np.matmul(P, V), atol=1e-11)
    assert np.allclose(W, W0 + np.einsum("bhti,bht,bhtj->bhij", K, eta, V), atol=1e-11)


# ---------------------------------------------------------------------------
# P-2: hand-derived gradients vs autograd and finite differences
# ---------------------------------------------------------------------------

def torch_linear_loss(K, V, eta, W):
    return -(eta * ((K @ W) * V).sum(-1)).sum(-1)


def torch_swiglu_loss(K, V, eta, W1, W3, W2):
    f = (torch.nn.functional.silu(K @ W1) * (K @ W3)) @ W2
    return -(eta * (f * V).sum(-1)).sum(-1)


def check_linear_grad(grad_fn=TO.linear_binding_grad, seed=0):
    Q, K, V, eta, W0 = rand_case(B=2, H=2, T=5, dk=4, dv=3, seed=seed)
    Wt = torch.tensor(W0, requires_grad=True)
    torch_linear_loss(*map(torch.tensor, (K, V, eta)), Wt).sum().backward()
    g = grad_fn(K, V, eta, W0)
    ok = np.allclose(g, Wt.grad.numpy(), atol=1e-12)
    # central differences on the oracle's own loss (independent of torch)
    h = 1e-6
    fd = np.zeros_like(W0)
    for idx in np.ndindex(W0.shape):
        Wp, Wm = W0.copy(), W0.copy()
        Wp[idx] += h
        Wm[idx] -= h
        b, hh = idx[0], idx[1]
        fd[idx] = (TO.linear_binding_loss(K, V, eta, Wp)[b, hh]
                   - TO.linear_binding_loss(K, V, eta, Wm)[b, hh]) / (2 * h)
    ok &= np.allclose(g, fd, atol=1e-7)
    return bool(ok)


def check_swiglu_grad(grad_fn=TO.swiglu_binding_grad, seed=0):
    Q, K, V, eta, W1, W3, W2 = rand_swiglu(B=1, H=2, T=5, d=3, dh=4, seed=seed)
    ws = [torch.tensor(w, requires_grad=True) for w in (W1, W3, W2)]
    torch_swiglu_loss(*map(torch.tensor, (K, V, eta)), *ws).sum().backward()
    g1, g3, g2 = grad_fn(K, V, eta, W1, W3, W2)
    ok = True
    for g, w in zip((g1, g3, g2), ws):
        ok &= np.allclose(g, w.grad.numpy(), atol=1e-12)
    h = 1e-6
    for which, (g, W) in enumerate(zip((g1, g3, g2), (W1, W3, W2))):
        for idx in np.ndindex(W.shape):
            Wp, Wm = W.copy(), W.copy()
            Wp[idx] += h
            Wm[idx] -= h
            args_p = [W1, W3, W2]
            args_m = [W1, W3, W2]
            args_p[which], args_m[which] = Wp, Wm
            fd = (TO.swiglu_binding_loss(K, V, eta, *args_p)[idx[0], idx[1]]
                  - TO.swiglu_binding_loss(K, V, eta, *args_m)[idx[0], idx[1]]) / (2 * h)
            ok &= abs(g[idx] - fd) < 1e-7
    return bool(ok)


def test_p2_linear_gradient():
    assert check_linear_grad()


def test_p2_swiglu_gradient():
    assert check_swiglu_grad(seed=0)
    assert check_swiglu_grad(seed=1)


def test_silu_prime_matches_autograd():
    a = torch.linspace(-8, 8, 101, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.silu(a).sum().backward()
    assert np.allclose(TO.silu_prime(a.detach().numpy()), a.grad.numpy(), atol=1e-14)
    assert np.allclose(TO.silu(a.detach().numpy()),
                       torch.nn.functional.silu(a).detach().numpy(), atol=1e-14)


# ---------------------------------------------------------------------------
# P-4: special cases
# ---------------------------------------------------------------------------

def test_p4_zero_eta_reads_initial_state():
    Q, K, V, eta, W0 = rand_case(seed=4)
    O, W = TO.per_token_linear(Q, K, V, 0 * eta, W0)
    assert np.allclose(O, Q @ W0, atol=1e-13) and np.array_equal(W, W0)


def test_p4_variant6_textbook_causal_linear_attention():
    # W0 = 0 and eta = 1: standard causal linear attention tril(Q K^T) V.
    Q, K, V, eta, W0 = rand_case(B=1, H=1, T=11, dk=3, dv=2, seed=5)
    O, _ = TO.per_token_linear(Q, K, V, np.ones_like(eta), 0 * W0)
    T = Q.shape[2]
    ref = np.zeros_like(O)
    for t in range(T):
        for i in range(t + 1):
            ref[0, 0, t] += float(np.dot(Q[0, 0, t], K[0, 0, i])) * V[0, 0, i]
    assert np.allclose(O, ref, atol=1e-12)


def test_p4_gradient_ascent_flips_the_accumulated_term():
    Q, K, V, eta, W0 = rand_case(seed=6)
    Op, Wp = TO.per_token_linear(Q, K, V, eta, W0)
    Om, Wm = TO.per_token_linear(Q, K, V, -eta, W0)
    base = Q @ W0
    assert np.allclose(Om - base, -(Op - base), atol=1e-12)
    assert np.allclose(Wm - W0, -(Wp - W0), atol=1e-12)


def test_p4_single_token():
    Q, K, V, eta, W0 = rand_case(T=1, seed=7)
    O, W = TO.per_token_linear(Q, K, V, eta, W0)
    Wref = W0 + eta[:, :, 0, None, None] * K[:, :, 0, :, None] * V[:, :, 0, None, :]
    assert np.allclose(W, Wref, atol=1e-14)
    assert np.allclose(O[:, :, 0], np.einsum("bhi,bhij->bhj", Q[:, :, 0], Wref), atol=1e-14)


def test_p4_queries_replaced_by_keys():
    Q, K, V, eta, W0 = rand_case(seed=8)
    O, _ = TO.per_token_linear(K, K, V, eta, W0)
    assert np.allclose(O, brute_force_linear_attention(K, K, V, eta, W0), atol=1e-12)


def test_p4_repeated_token_with_split_rate():
    # n GD steps of rate eta/n on the same token equal one step of rate eta
    # (the linear gradient does not depend on W).
    Q, K, V, eta, W0 = rand_case(B=1, H=1, T=4, seed=9)
    n = 3
    rep = lambda X: np.repeat(X, n, axis=2)  # noqa: E731
    O1, W1 = TO.per_token_linear(Q, K, V, eta, W0)
    On, Wn = TO.per_token_linear(rep(Q), rep(K), rep(V), rep(eta) / n, W0)
    assert np.allclose(W1, Wn, atol=1e-13)
    assert np.allclose(O1, On[:, :, n - 1::n], atol=1e-13)


def test_p4_lact_fixed_point_with_unit_columns_and_zero_rate():
    Q, K, V, eta, W0 = rand_case(seed=10)
    W0 = W0 / np.linalg.norm(W0, axis=-2, keepdims=True)
    O, W = TO.large_chunk_linear(Q, K, V, 0 * eta, W0, 4)
    assert np.allclose(O, Q @ W0, atol=1e-13) and np.allclose(W, W0, atol=1e-14)


# ---------------------------------------------------------------------------
# P-5: large-chunk linear closed forms and invariants
# ---------------------------------------------------------------------------

def test_p5_single_chunk():
    Q, K, V, eta, W0 = rand_case(seed=11)
    T = Q.shape[2]
    O, W = TO.large_chunk_linear(Q, K, V, eta, W0, T)
    assert np.allclose(O, Q @ W0, atol=1e-13)
    M = W0 + np.einsum("bhti,bht,bhtj->bhij", K, eta, V)
    assert np.allclose(W, M / np.linalg.norm(M, axis=-2, keepdims=True), atol=1e-13)


@pytest.mark.parametrize("chunk", [1, 3, 4, 13, 20])
def test_p5_unnormalised_is_block_causal_linear_attention(chunk):
    Q, K, V, eta, W0 = rand_case(seed=12)
    T = Q.shape[2]
    O, _ = TO.large_chunk_linear(Q, K, V, eta, W0, chunk, normalize=False)
    c = np.arange(T) // chunk
    mask = (c[None, :] < c[:, None]).astype(np.float64)          # strictly earlier chunks
    P = np.matmul(Q, np.swapaxes(K, -1, -2)) * mask * eta[:, :, None, :]
    assert np.allclose(O, Q @ W0 + P @ V, atol=1e-11)
    if chunk == 1:
        Oex, _ = TO.per_token_linear(Q, K, V, eta, W0, inclusive=False)
        assert np.allclose(O, Oex, atol=1e-12)


@pytest.mark.parametrize("chunk", [2, 5, 13])
def test_p5_unit_columns_after_every_update(chunk):
    Q, K, V, eta, W0 = rand_case(seed=13)
    T = Q.shape[2]
    for stop in range(chunk, T + chunk, chunk):
        _, W = TO.large_chunk_linear(Q[:, :, :stop], K[:, :, :stop], V[:, :, :stop],
                                     eta[:, :, :stop], W0, chunk)
        assert np.allclose(np.linalg.norm(W, axis=-2), 1.0, atol=1e-13)


def test_normalize_columns_zero_column_uses_eps_floor():
    W = np.zeros((1, 1, 3, 2))
    W[0, 0, :, 0] = [3.0, 4.0, 0.0]
    out = TO.normalize_columns(W)
    assert np.allclose(out[0, 0, :, 0], [0.6, 0.8, 0.0]) and np.all(out[0, 0, :, 1] == 0)


# ---------------------------------------------------------------------------
# P-6: SwiGLU reductions
# ---------------------------------------------------------------------------

def torch_mlp(X, W1, W3, W2):
    t = lambda a: torch.tensor(a)  # noqa: E731
    return ((torch.nn.functional.silu(t(X) @ t(W1)) * (t(X) @ t(W3))) @ t(W2)).numpy()


def test_p6_single_chunk_is_mlp_forward_then_one_normalised_step():
    Q, K, V, eta, W1, W3, W2 = rand_swiglu(seed=14)
    T = Q.shape[2]
    O, (N1, N3, N2) = TO.large_chunk_swiglu(Q, K, V, eta, W1, W3, W2, T)
    assert np.allclose(O, torch_mlp(Q, W1, W3, W2), atol=1e-12)
    ws = [torch.tensor(w, requires_grad=True) for w in (W1, W3, W2)]
    torch_swiglu_loss(*map(torch.tensor, (K, V, eta)), *ws).sum().backward()
    for new, w in zip((N1, N3, N2), ws):
        step = w.detach().numpy() - w.grad.numpy()
        assert np.allclose(new, step / np.linalg.norm(step, axis=-2, keepdims=True), atol=1e-12)
        assert np.allclose(np.linalg.norm(new, axis=-2), 1.0, atol=1e-13)


@pytest.mark.parametrize("chunk", [1, 3, 10])
def test_p6_last_layer_only_is_linear_attention_in_feature_space(chunk):
    Q, K, V, eta, W1, W3, W2 = rand_swiglu(seed=15)
    T = Q.shape[2]
    O, (_, _, W2T) = TO.large_chunk_swiglu(Q, K, V, eta, W1, W3, W2, chunk,
                                           normalize=False, update_w1w3=False)
    phi = lambda X: (torch.nn.functional.silu(torch.tensor(X) @ torch.tensor(W1))  # noqa: E731
                     * (torch.tensor(X) @ torch.tensor(W3))).numpy()
    fq, fk = phi(Q), phi(K)
    c = np.arange(T) // chunk
    mask = (c[None, :] < c[:, None]).astype(np.float64)
    P = np.matmul(fq, np.swapaxes(fk, -1, -2)) * mask * eta[:, :, None, :]
    assert np.allclose(O, fq @ W2 + P @ V, atol=1e-11)
    assert np.allclose(W2T, W2 + np.einsum("bhti,bht,bhtj->bhij", fk, eta, V), atol=1e-11)


# ---------------------------------------------------------------------------
# Ordering variant: a chunk updates, then reads (LaCT review, read-order section)
# ---------------------------------------------------------------------------

def test_update_first_linear_single_chunk():
    Q, K, V, eta, W0 = rand_case(seed=21)
    T = Q.shape[2]
    O, W = TO.large_chunk_linear(Q, K, V, eta, W0, T, read_first=False)
    M = W0 + np.einsum("bhti,bht,bhtj->bhij", K, eta, V)
    Mn = M / np.linalg.norm(M, axis=-2, keepdims=True)
    assert np.allclose(W, Mn, atol=1e-13)
    assert np.allclose(O, Q @ Mn, atol=1e-13)


@pytest.mark.parametrize("chunk", [1, 3, 4, 13, 20])
def test_update_first_unnormalised_is_inclusive_block_linear_attention(chunk):
    Q, K, V, eta, W0 = rand_case(seed=22)
    T = Q.shape[2]
    O, _ = TO.large_chunk_linear(Q, K, V, eta, W0, chunk, normalize=False, read_first=False)
    c = np.arange(T) // chunk
    mask = (c[None, :] <= c[:, None]).astype(np.float64)         # earlier chunks and the own chunk
    P = np.matmul(Q, np.swapaxes(K, -1, -2)) * mask * eta[:, :, None, :]
    assert np.allclose(O, Q @ W0 + P @ V, atol=1e-11)
    if chunk == 1:
        Oin, _ = TO.per_token_linear(Q, K, V, eta, W0, inclusive=True)
        assert np.allclose(O, Oin, atol=1e-12)


@pytest.mark.parametrize("chunk", [1, 3, 10])
def test_update_first_leaves_the_state_sequence_unchanged(chunk):
    Q, K, V, eta, W0 = rand_case(seed=23)
    _, Wa = TO.large_chunk_linear(Q, K, V, eta, W0, chunk)
    _, Wb = TO.large_chunk_linear(Q, K, V, eta, W0, chunk, read_first=False)
    assert np.array_equal(Wa, Wb)
    Q, K, V, eta, W1, W3, W2 = rand_swiglu(seed=24)
    _, Sa = TO.large_chunk_swiglu(Q, K, V, eta, W1, W3, W2, chunk)
    _, Sb = TO.large_chunk_swiglu(Q, K, V, eta, W1, W3, W2, chunk, read_first=False)
    for a, b in zip(Sa, Sb):
        assert np.array_equal(a, b)


def test_update_first_swiglu_single_chunk_reads_the_stepped_weights():
    Q, K, V, eta, W1, W3, W2 = rand_swiglu(seed=25)
    T = Q.shape[2]
    O, (N1, N3, N2) = TO.large_chunk_swiglu(Q, K, V, eta, W1, W3, W2, T, read_first=False)
    ws = [torch.tensor(w, requires_grad=True) for w in (W1, W3, W2)]
    torch_swiglu_loss(*map(torch.tensor, (K, V, eta)), *ws).sum().backward()
    stepped = []
    for w in ws:
        st = w.detach().numpy() - w.grad.numpy()
        stepped.append(st / np.linalg.norm(st, axis=-2, keepdims=True))
    for new, ref in zip((N1, N3, N2), stepped):
        assert np.allclose(new, ref, atol=1e-12)
    assert np.allclose(O, torch_mlp(Q, *stepped), atol=1e-12)


@pytest.mark.parametrize("chunk", [1, 3, 10])
def test_update_first_swiglu_last_layer_only_is_inclusive_feature_attention(chunk):
    Q, K, V, eta, W1, W3, W2 = rand_swiglu(seed=26)
    T = Q.shape[2]
    O, _ = TO.large_chunk_swiglu(Q, K, V, eta, W1, W3, W2, chunk, normalize=False, update_w1w3=False,
                                 read_first=False)
    phi = lambda X: (torch.nn.functional.silu(torch.tensor(X) @ torch.tensor(W1))  # noqa: E731
                     * (torch.tensor(X) @ torch.tensor(W3))).numpy()
    fq, fk = phi(Q), phi(K)
    c = np.arange(T) // chunk
    mask = (c[None, :] <= c[:, None]).astype(np.float64)
    P = np.matmul(fq, np.swapaxes(fk, -1, -2)) * mask * eta[:, :, None, :]
    assert np.allclose(O, fq @ W2 + P @ V, atol=1e-11)


def test_variant_mode_names_dispatch():
    Q, K, V, eta, W0 = rand_case(seed=27)
    O1, W1 = oracle.forward(Q, K, V, eta, W0, 5, "per_token_linear_exclusive")
    O2, W2 = TO.per_token_linear(Q, K, V, eta, W0, inclusive=False)
    assert np.array_equal(O1, O2) and np.array_equal(W1, W2)
    O1, W1 = oracle.forward(Q, K, V, eta, W0, 5, "large_chunk_linear_update_first")
    O2, W2 = TO.large_chunk_linear(Q, K, V, eta, W0, 5, read_first=False)
    assert np.array_equal(O1, O2) and np.array_equal(W1, W2)
    Q, K, V, eta, A1, A3, A2 = rand_swiglu(seed=28)
    Wp = TO.swiglu_pack(A1, A3, A2)
    O1, Wf = oracle.forward(Q, K, V, eta, Wp, 3, "large_chunk_swiglu_update_first", d_h=6)
    O2, Ws = TO.large_chunk_swiglu(Q, K, V, eta, A1, A3, A2, 3, read_first=False)
    assert np.array_equal(O1, O2) and np.array_equal(Wf, TO.swiglu_pack(*Ws))


def test_swiglu_pack_roundtrip_and_dispatch():
    Q, K, V, eta, W1, W3, W2 = rand_swiglu(seed=16)
    Wp = TO.swiglu_pack(W1, W3, W2)
    for a, b in zip(TO.swiglu_unpack(Wp, 4, 6), (W1, W3, W2)):
        assert np.array_equal(a, b)
    O1, Wf = oracle.forward(Q, K, V, eta, Wp, 3, "large_chunk_swiglu", d_h=6)
    O2, Ws = TO.large_chunk_swiglu(Q, K, V, eta, W1, W3, W2, 3)
    assert np.array_equal(O1, O2) and np.array_equal(Wf, TO.swiglu_pack(*Ws))


# ---------------------------------------------------------------------------
# P-7: the state is the checkpoint (resume)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode,chunk,t1", [
    ("per_token_linear", 4, 5), ("large_chunk_linear", 4, 8), ("large_chunk_swiglu", 3, 6)])
def test_p7_resume(mode, chunk, t1):
    if mode == "large_chunk_swiglu":
        Q, K, V, eta, W1, W3, W2 = rand_swiglu(T=12, seed=17)
        W0 = TO.swiglu_pack(W1, W3, W2)
    else:
        Q, K, V, eta, W0 = rand_case(T=12, seed=17)
    kw = dict(chunk=chunk, mode=mode, d_h=6)
    O, W = oracle.forward(Q, K, V, eta, W0, **kw)
    O1, Wm = oracle.forward(Q[:, :, :t1], K[:, :, :t1], V[:, :, :t1], eta[:, :, :t1], W0, **kw)
    O2, W2_ = oracle.forward(Q[:, :, t1:], K[:, :, t1:], V[:, :, t1:], eta[:, :, t1:], Wm, **kw)
    assert np.allclose(np.concatenate([O1, O2], axis=2), O, atol=1e-12)
    assert np.allclose(W2_, W, atol=1e-12)


# ---------------------------------------------------------------------------
# Input recipe sanity (the generator holds no method arithmetic)
# ---------------------------------------------------------------------------

def test_workload_generator_recipe():
    s = workloads.make_spec("per_token_linear", 2, 2, 7, 8, dtype="bf16", eta="sigmoid")
    a = workloads.generate(s, seed=0)
    b = workloads.generate(s, seed=0)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert np.allclose(np.linalg.norm(a["Q"].astype(np.float64), axis=-1), 1, atol=1e-2)
    assert np.array_equal(workloads.bf16_round(a["V"]), a["V"])
    assert np.all((a["eta"] > 0) & (a["eta"] < 0.1))
    assert np.array_equal(a["W0"][0], a["W0"][1])          # one draw per head, shared over B
    assert not np.array_equal(a["W0"][0, 0], a["W0"][0, 1])


def test_bf16_round_ties_to_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9], dtype=np.float32)
    r = workloads.bf16_round(x)
    ref = torch.tensor(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(r, ref)


# ---------------------------------------------------------------------------
# Mutation tests: each planted mistake must be caught by a pin
# ---------------------------------------------------------------------------

def _pt_transposed(Q, K, V, eta, W0, inclusive=True):
    W = W0.copy()
    O = np.zeros(Q.shape[:-1] + (V.shape[-1],))
    for t in range(Q.shape[2]):
        W = W + eta[:, :, t, None, None] * V[:, :, t, :, None] * K[:, :, t, None, :]
        O[:, :, t] = np.einsum("bhi,bhij->bhj", Q[:, :, t], W)
    return O, W


def _pt_wrong_sign(Q, K, V, eta, W0, inclusive=True):
    return TO.per_token_linear(Q, K, V, -eta, W0, inclusive)


def _pt_always_exclusive(Q, K, V, eta, W0, inclusive=True):
    return TO.per_token_linear(Q, K, V, eta, W0, inclusive=False)


def _lcl_rows(Q, K, V, eta, W0, chunk, normalize=True):
    W = W0.copy()
    O = np.zeros(Q.shape[:-1] + (V.shape[-1],))
    for s in range(0, Q.shape[2], chunk):
        e = min(s + chunk, Q.shape[2])
        O[:, :, s:e] = Q[:, :, s:e] @ W
        W = W - TO.linear_binding_grad(K[:, :, s:e], V[:, :, s:e], eta[:, :, s:e])
        W = W / np.linalg.norm(W, axis=-1, keepdims=True)          # wrong axis
    return O, W


def _lcl_update_then_read(Q, K, V, eta, W0, chunk, normalize=True):
    W = W0.copy()
    O = np.zeros(Q.shape[:-1] + (V.shape[-1],))
    for s in range(0, Q.shape[2], chunk):
        e = min(s + chunk, Q.shape[2])
        W = TO.normalize_columns(W - TO.linear_binding_grad(K[:, :, s:e], V[:, :, s:e], eta[:, :, s:e]))
        O[:, :, s:e] = Q[:, :, s:e] @ W
    return O, W


def _swiglu_grad_sigmoid_not_silu_prime(K, V, eta, W1, W3, W2):
    a = K @ W1
    b = K @ W3
    dy = -eta[..., None] * V
    dh = dy @ np.swapaxes(W2, -1, -2)
    s = 1 / (1 + np.exp(-a))
    h = TO.silu(a) * b
    Kt = np.swapaxes(K, -1, -2)
    return Kt @ (dh * b * s), Kt @ (dh * TO.silu(a)), np.swapaxes(h, -1, -2) @ dy


def _swiglu_grad_dropped_w2_term(K, V, eta, W1, W3, W2):
    g1, g3, g2 = TO.swiglu_binding_grad(K, V, eta, W1, W3, W2)
    return g1, g3, 0 * g2


def _linear_grad_missing_eta(K, V, eta, W=None):
    return -np.swapaxes(K, -1, -2) @ V


@pytest.mark.parametrize("mutant", [_pt_transposed, _pt_wrong_sign, _pt_always_exclusive])
def test_mutants_per_token_are_caught(mutant):
    assert not (check_golden(pt=mutant) and check_closed_form(pt=mutant))


@pytest.mark.parametrize("mutant", [_lcl_rows, _lcl_update_then_read])
def test_mutants_large_chunk_are_caught(mutant):
    assert not check_golden(lcl=mutant)


@pytest.mark.parametrize("mutant", [_swiglu_grad_sigmoid_not_silu_prime, _swiglu_grad_dropped_w2_term])
def test_mutants_swiglu_grad_are_caught(mutant):
    assert not check_swiglu_grad(grad_fn=mutant)


def test_mutant_linear_grad_is_caught():
    assert not check_linear_grad(grad_fn=_linear_grad_missing_eta)


def test_last_layer_mode_dispatch_is_the_feature_space_form():
    # the product mode's name dispatches to the pinned last-layer-only, unnormalised function
    Q, K, V, eta, W1, W3, W2 = rand_swiglu(seed=19)
    d, dh = W1.shape[-2], W1.shape[-1]
    O, Wp = TO.forward(Q, K, V, eta, TO.swiglu_pack(W1, W3, W2), 3, "large_chunk_swiglu_last_layer", d_h=dh)
    O2, (W1b, W3b, W2b) = TO.large_chunk_swiglu(Q, K, V, eta, W1, W3, W2, 3, normalize=False, update_w1w3=False)
    assert np.array_equal(O, O2)
    assert np.array_equal(Wp, TO.swiglu_pack(W1, W3, W2b))
    assert np.array_equal(W1b, W1) and np.array_equal(W3b, W3)



# ---------------------------------------------------------------------------
# Large-chunk linear with momentum (LaCT review, non-linear-memory section)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("read_first", [True, False])
def test_momentum_zero_is_the_plain_method(read_first):
    Q, K, V, eta, W0 = rand_case(seed=31)
    O, W = TO.large_chunk_linear(Q, K, V, eta, W0, 4, read_first=read_first)
    Om, Wm, M = TO.large_chunk_linear(Q, K, V, eta, W0, 4, read_first=read_first, momentum=0.0)
    assert np.array_equal(O, Om) and np.array_equal(W, Wm)
    last = slice(12, 13)                                   # T = 13: the last chunk holds one token
    assert np.allclose(M, np.swapaxes(K[:, :, last], -1, -2) @ (eta[:, :, last, None] * V[:, :, last]))


def test_momentum_two_chunks_by_hand():
    Q, K, V, eta, W0 = rand_case(T=8, seed=32)
    beta = 0.7
    D0 = np.swapaxes(K[:, :, :4], -1, -2) @ (eta[:, :, :4, None] * V[:, :, :4])
    D1 = np.swapaxes(K[:, :, 4:], -1, -2) @ (eta[:, :, 4:, None] * V[:, :, 4:])
    n = lambda X: X / np.linalg.norm(X, axis=-2, keepdims=True)  # noqa: E731
    W1 = n(W0 + D0)
    W2 = n(W1 + beta * D0 + D1)
    O, W, M = TO.large_chunk_linear(Q, K, V, eta, W0, 4, momentum=beta)
    assert np.allclose(O[:, :, :4], Q[:, :, :4] @ W0) and np.allclose(O[:, :, 4:], Q[:, :, 4:] @ W1)
    assert np.allclose(W, W2) and np.allclose(M, beta * D0 + D1)


@pytest.mark.parametrize("beta", [0.5, 0.9])
def test_momentum_unnormalised_is_a_discounted_sum(beta):
    # without the normalisation W_T = W0 + sum_c M_c with M_c = sum_{c' <= c} beta^(c - c') D_c'
    Q, K, V, eta, W0 = rand_case(T=13, seed=33)
    Ds = [np.swapaxes(K[:, :, s:s + 3], -1, -2) @ (eta[:, :, s:s + 3, None] * V[:, :, s:s + 3]) for s in range(0, 13, 3)]
    Ms = [sum(beta ** (c - k) * Ds[k] for k in range(c + 1)) for c in range(len(Ds))]
    _, W, M = TO.large_chunk_linear(Q, K, V, eta, W0, 3, normalize=False, momentum=beta)
    assert np.allclose(W, W0 + sum(Ms)) and np.allclose(M, Ms[-1])


@pytest.mark.parametrize("read_first", [True, False])
def test_momentum_resume_with_the_buffer(read_first):
    Q, K, V, eta, W0 = rand_case(T=13, seed=34)
    O, W, M = TO.large_chunk_linear(Q, K, V, eta, W0, 3, read_first=read_first, momentum=0.8)
    Oa, Wa, Ma = TO.large_chunk_linear(Q[:, :, :6], K[:, :, :6], V[:, :, :6], eta[:, :, :6], W0, 3,
                                       read_first=read_first, momentum=0.8)
    Ob, Wb, Mb = TO.large_chunk_linear(Q[:, :, 6:], K[:, :, 6:], V[:, :, 6:], eta[:, :, 6:], Wa, 3,
                                       read_first=read_first, momentum=0.8, M0=Ma)
    assert np.allclose(np.concatenate([Oa, Ob], axis=2), O) and np.allclose(Wb, W) and np.allclose(Mb, M)
