"""Plain fp64 CPU oracle for the TTT-with-KV-binding forward pass, its update rules and its backward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or
links this module: only the tests, the smoke check and the CPU-baseline leg
of the benchmark do. It shares no code with the HIP library.

What it computes (sources are the pages on "Test-Time Training with KV
Binding Is Secretly Linear Attention" and on LaCT, "Test-Time Training Done
Right"; no page prints an equation, so each step below restates in symbols
what the cited passage says in words):

* A fast weight ``W`` is a small model ``f_W``.  Each token ``i`` carries a
  key ``k_i``, a value ``v_i``, a query ``q_i`` and a learning rate
  ``eta_i``.  The inner-loop (binding) loss for a token is the negative inner
  product ``L_i(W) = -<f_W(k_i), v_i>`` (LaCT review, section on non-linear
  memory and local attention).  An update is one explicit gradient-descent
  step ``W <- W - eta * dL/dW``; a negative ``eta`` is gradient ascent (paper
  summary, technical section 2A item 4 and section 3 item 2).
* Per-token mode (paper summary, technical section 2B; podcast at 7:50 to
  9:01): a linear ``f_W(k) = k W`` gets one step per token and the query reads
  the memory.  The read is taken after the token's own update, so the closed
  form is ``o_t = q_t (W0 + sum_{i<=t} eta_i k_i^T v_i)``; ``inclusive=False``
  gives the read-before-update variant ``sum_{i<t}``.
* Large-chunk modes (LaCT review, sections on fast weights, on non-linear
  memory, and on read order): tokens are grouped in chunks; every token of a
  chunk reads the memory left by the previous chunks, then one summed,
  eta-weighted gradient step is applied for the whole chunk and the weights
  are L2-normalised after the update.  Memory is either a linear map or a
  SwiGLU MLP with three matrices.  ``read_first=False`` gives the
  update-then-read order the LaCT review's read-order section describes for
  posed-image view synthesis (the input set is absorbed, then queried),
  applied chunk by chunk: a chunk first updates and normalises the weights,
  then its queries read the result.

Readings taken where the pages are silent:
row-vector convention ``o = q W`` with ``W`` stored ``[d_in, d_out]``; the
post-update normalisation gives every output unit's fan-in vector (a column
of the ``[d_in, d_out]`` store) unit L2 norm, dividing by
``max(norm, 1e-12)``; the initial weights are not normalised before the
first read; the SwiGLU branch with SiLU is ``x W1``; all SwiGLU gradients of
a chunk are taken at the weights that read that chunk; a shorter final chunk
follows the same read-then-update order.

Arrays are float64 numpy arrays.  Shapes: Q, K ``[B,H,T,d_k]``; V
``[B,H,T,d_v]``; eta ``[B,H,T]``; linear W ``[B,H,d_k,d_v]``; SwiGLU
W1, W3 ``[B,H,d,d_h]`` and W2 ``[B,H,d_h,d]``.  All (b, h) pairs are
independent, so every function is vectorised over them only; the token and
chunk loops are explicit and sequential.
"""
from __future__ import annotations

import numpy as np

NORM_EPS = 1e-12


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Inner-loop losses and their hand-derived gradients
# ---------------------------------------------------------------------------

def linear_binding_loss(K, V, eta, W):
    """``sum_i eta_i * (-<k_i W, v_i>)`` per (b, h): the eta-weighted
    negative inner-product binding loss of a linear fast weight (LaCT review,
    non-linear memory section).  Returns ``[B,H]``."""
    K, V, eta, W = map(_f64, (K, V, eta, W))
    pred = np.matmul(K, W)                      # f_W(k_i) = k_i W
    return -np.sum(eta * np.sum(pred * V, axis=-1), axis=-1)


def linear_binding_grad(K, V, eta, W=None):
    """Gradient of :func:`linear_binding_loss` with respect to W.

    d/dW_{ab} of ``-sum_i eta_i sum_j (sum_a k_ia W_aj) v_ij`` is
    ``-sum_i eta_i k_ia v_ib``: it does not depend on W.  Returned as
    ``[B,H,d_k,d_v]``."""
    K, V, eta = map(_f64, (K, V, eta))
    return -np.matmul(np.swapaxes(K * eta[..., None], -1, -2), V)


def silu(a):
    """SiLU ``a * sigmoid(a)``."""
    return a / (1.0 + np.exp(-a))


def silu_prime(a):
    """Derivative of SiLU: ``s (1 + a (1 - s))`` with ``s = sigmoid(a)``."""
    s = 1.0 / (1.0 + np.exp(-a))
    return s * (1.0 + a * (1.0 - s))


def swiglu_forward(X, W1, W3, W2):
    """SwiGLU fast-weight MLP ``f_W(x) = (silu(x W1) * (x W3)) W2`` (LaCT
    review: the usual memory is a SwiGLU MLP with three matrices)."""
    X, W1, W3, W2 = map(_f64, (X, W1, W3, W2))
    return np.matmul(silu(np.matmul(X, W1)) * np.matmul(X, W3), W2)


def swiglu_binding_loss(K, V, eta, W1, W3, W2):
    """``sum_i eta_i * (-<f_W(k_i), v_i>)`` per (b, h), returns ``[B,H]``."""
    pred = swiglu_forward(K, W1, W3, W2)
    return -np.sum(_f64(eta) * np.sum(pred * _f64(V), axis=-1), axis=-1)


def swiglu_binding_grad(K, V, eta, W1, W3, W2):
    """Hand-derived gradient of :func:`swiglu_binding_loss`.

    With ``a = k W1``, ``b = k W3``, ``h = silu(a) * b`` and ``y = h W2``,
    the loss is ``-sum_i eta_i <y_i, v_i>``.  Back-propagation by hand:
    ``dL/dy_i = -eta_i v_i``; ``dL/dW2 = sum_i h_i^T dL/dy_i``;
    ``dL/dh_i = dL/dy_i W2^T``; ``dL/da_i = dL/dh_i * b_i * silu'(a_i)``;
    ``dL/db_i = dL/dh_i * silu(a_i)``; ``dL/dW1 = sum_i k_i^T dL/da_i``;
    ``dL/dW3 = sum_i k_i^T dL/db_i``.  Returns (dW1, dW3, dW2)."""
    K, V, eta, W1, W3, W2 = map(_f64, (K, V, eta, W1, W3, W2))
    a = np.matmul(K, W1)
    b = np.matmul(K, W3)
    h = silu(a) * b
    dy = -eta[..., None] * V
    dW2 = np.matmul(np.swapaxes(h, -1, -2), dy)
    dh = np.matmul(dy, np.swapaxes(W2, -1, -2))
    da = dh * b * silu_prime(a)
    db = dh * silu(a)
    Kt = np.swapaxes(K, -1, -2)
    return np.matmul(Kt, da), np.matmul(Kt, db), dW2


def normalize_columns(W):
    """Give every column (one output unit's fan-in vector over the
    second-to-last axis) unit L2 norm, dividing by ``max(norm, 1e-12)``
    (LaCT review: L2 normalisation after the weight update)."""
    n = np.sqrt(np.sum(W * W, axis=-2, keepdims=True))
    return W / np.maximum(n, NORM_EPS)


# ---------------------------------------------------------------------------
# The three forward modes
# ---------------------------------------------------------------------------

def per_token_linear(Q, K, V, eta, W0, inclusive=True):
    """Per-token TTT with a linear fast weight: for t = 0..T-1 take one
    gradient step on token t's binding loss, and let q_t read the memory
    (after the step when ``inclusive``, else before it).

    Paper summary, technical section 2B (TTT rewritten exactly as learned
    linear attention); podcast at 7:50 (output is the query times a running
    sum of key-value products).  Returns (O ``[B,H,T,d_v]``, W_T)."""
    Q, K, V, eta, W = map(_f64, (Q, K, V, eta, W0))
    W = W.copy()
    B, H, T, _ = Q.shape
    O = np.zeros(Q.shape[:-1] + (V.shape[-1],))
    for t in range(T):
        k = K[:, :, t:t + 1, :]
        v = V[:, :, t:t + 1, :]
        e = eta[:, :, t:t + 1]
        if not inclusive:
            O[:, :, t, :] = np.matmul(Q[:, :, t:t + 1, :], W)[:, :, 0, :]
        g = linear_binding_grad(k, v, np.ones_like(e))   # -k_t^T v_t
        W = W - e[..., None] * g                          # GD step, rate eta_t
        if inclusive:
            O[:, :, t, :] = np.matmul(Q[:, :, t:t + 1, :], W)[:, :, 0, :]
    return O, W


def per_token_linear_backward(Q, K, V, eta, W0, dO, dW_T, inclusive=True):
    """Reverse-mode gradients of :func:`per_token_linear`: given the
    upstream gradients ``dO`` (of O) and ``dW_T`` (of the final memory),
    return ``(dQ, dK, dV, deta, dW0)``.

    Training the outer model through the per-token inner loop (the paper
    summary reports training speed-ups of the parallel form, technical
    section 4; podcast at 14:17) needs these.  They are derived by hand from
    the token loop, walked backwards: the forward step is
    ``W_t = W_{t-1} + eta_t k_t^T v_t`` and the read is ``o_t = q_t W_t``
    (``W_{t-1}`` when not ``inclusive``).  With ``G`` the gradient with
    respect to the current memory (``dW_T`` at the end):
      read:  ``dq_t = dO_t W^T`` for the memory the query read, and
             ``G += q_t^T dO_t``;
      step:  ``deta_t = <G, k_t^T v_t> = k_t G v_t^T``,
             ``dk_t = eta_t v_t G^T``, ``dv_t = eta_t k_t G``;
             the memory before the step receives ``G`` unchanged.
    Memories are recovered exactly in reverse by undoing the steps from the
    final one.  ``dW0`` is ``G`` after the first token."""
    Q, K, V, eta, W0, dO, dW_T = map(_f64, (Q, K, V, eta, W0, dO, dW_T))
    _, W = per_token_linear(Q, K, V, eta, W0, inclusive=inclusive)
    G = dW_T.copy()
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    deta = np.zeros_like(eta)
    T = Q.shape[2]
    for t in range(T - 1, -1, -1):
        q, k, v = Q[:, :, t:t + 1, :], K[:, :, t:t + 1, :], V[:, :, t:t + 1, :]
        do = dO[:, :, t:t + 1, :]
        e = eta[:, :, t][..., None, None]
        if inclusive:                                     # o_t = q_t W_t
            dQ[:, :, t, :] = np.matmul(do, np.swapaxes(W, -1, -2))[:, :, 0, :]
            G = G + np.matmul(np.swapaxes(q, -1, -2), do)
        deta[:, :, t] = np.matmul(np.matmul(k, G), np.swapaxes(v, -1, -2))[:, :, 0, 0]
        dK[:, :, t, :] = (e * np.matmul(v, np.swapaxes(G, -1, -2)))[:, :, 0, :]
        dV[:, :, t, :] = (e * np.matmul(k, G))[:, :, 0, :]
        W = W - e * np.matmul(np.swapaxes(k, -1, -2), v)  # undo step t: W_{t-1}
        if not inclusive:                                 # o_t = q_t W_{t-1}
            dQ[:, :, t, :] = np.matmul(do, np.swapaxes(W, -1, -2))[:, :, 0, :]
            G = G + np.matmul(np.swapaxes(q, -1, -2), do)
    return dQ, dK, dV, deta, G


def large_chunk_linear_backward(Q, K, V, eta, W0, dO, dW_T, chunk, read_first=True):
    """Reverse-mode gradients of :func:`large_chunk_linear` (with the
    normalisation): ``(dQ, dK, dV, deta, dW0)`` from ``dO`` and ``dW_T``.

    Derived by hand from the chunk loop, walked backwards.  Chunk c forms
    ``P_c = W_{c-1} + K_c^T diag(eta_c) V_c`` and ``W_c = P_c / n_c`` per
    column, ``n_c = max(||P_c column||, 1e-12)``; its queries read
    ``R_c = W_{c-1}`` (``W_c`` when not ``read_first``).  With ``G`` the
    gradient of the newest memory (``dW_T`` at the end), for each chunk from
    the last:
      update-first read: ``dQ_c = dO_c W_c^T`` and ``G += Q_c^T dO_c``;
      normalisation: per column, ``dP = (G - w (w . G)) / n`` when the norm
      exceeds the floor (``w`` the normalised column), else ``G / 1e-12``;
      step: ``dK_c = diag(eta) V_c dP^T``, ``dV_c = diag(eta) K_c dP``,
      ``deta_t = k_t dP v_t^T``; the memory before the step gets ``dP``;
      read-first read: ``dQ_c = dO_c W_{c-1}^T`` and ``G = dP + Q_c^T dO_c``.
    ``dW0`` is ``G`` after the first chunk."""
    Q, K, V, eta, W0, dO, dW_T = map(_f64, (Q, K, V, eta, W0, dO, dW_T))
    T = Q.shape[2]
    starts = list(range(0, T, chunk))
    Ws = [W0.copy()]                     # W_{c-1} for every chunk, then W_T
    for s in starts:
        e = min(s + chunk, T)
        Ws.append(normalize_columns(Ws[-1] - linear_binding_grad(K[:, :, s:e], V[:, :, s:e], eta[:, :, s:e])))
    tr = lambda X: np.swapaxes(X, -1, -2)
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    deta = np.zeros_like(eta)
    G = dW_T.copy()
    for c in range(len(starts) - 1, -1, -1):
        s, e = starts[c], min(starts[c] + chunk, T)
        q, k, v, do = Q[:, :, s:e], K[:, :, s:e], V[:, :, s:e], dO[:, :, s:e]
        et = eta[:, :, s:e]
        if not read_first:
            dQ[:, :, s:e] = do @ tr(Ws[c + 1])
            G = G + tr(q) @ do
        P = Ws[c] + tr(k) @ (et[..., None] * v)
        n = np.sqrt(np.sum(P * P, axis=-2, keepdims=True))
        big = n > NORM_EPS
        w = P / np.maximum(n, NORM_EPS)
        dP = np.where(big, (G - w * np.sum(w * G, axis=-2, keepdims=True)) / np.maximum(n, NORM_EPS), G / NORM_EPS)
        dK[:, :, s:e] = et[..., None] * (v @ tr(dP))
        dV[:, :, s:e] = et[..., None] * (k @ dP)
        deta[:, :, s:e] = np.sum((k @ dP) * v, axis=-1)
        G = dP
        if read_first:
            dQ[:, :, s:e] = do @ tr(Ws[c])
            G = G + tr(q) @ do
    return dQ, dK, dV, deta, G


def silu_second(a):
    """Second derivative of SiLU: ``s (1 - s) (2 + a (1 - 2 s))`` with ``s = sigmoid(a)``."""
    s = 1.0 / (1.0 + np.exp(-a))
    return s * (1.0 - s) * (2.0 + a * (1.0 - 2.0 * s))


def swiglu_read_backward(X, W1, W3, W2, dY):
    """Reverse-mode gradients of ``Y = f_W(X)`` (the SwiGLU MLP) given ``dY``:
    ``(dX, (dW1, dW3, dW2))``.  With ``a = X W1``, ``b = X W3``,
    ``h = silu(a) b``: ``dh = dY W2^T``, ``dW2 = h^T dY``,
    ``da = dh b silu'(a)``, ``db = dh silu(a)``, ``dW1 = X^T da``,
    ``dW3 = X^T db``, ``dX = da W1^T + db W3^T``."""
    X, W1, W3, W2, dY = map(_f64, (X, W1, W3, W2, dY))
    tr = lambda M: np.swapaxes(M, -1, -2)  # noqa: E731
    a, b = X @ W1, X @ W3
    h = silu(a) * b
    dh = dY @ tr(W2)
    da = dh * b * silu_prime(a)
    db = dh * silu(a)
    return da @ tr(W1) + db @ tr(W3), (tr(X) @ da, tr(X) @ db, tr(h) @ dY)


def swiglu_step_vjp(K, V, eta, W1, W3, W2, D1, D3, D2):
    """Vector-Jacobian product of the chunk step ``S(W, K, V, eta) = sum_i
    eta_i grad_W <f_W(k_i), v_i>`` with the cotangent ``(D1, D3, D2)``.

    ``<(D1, D3, D2), S> = sum_i eta_i <ydot_i, v_i> =: phi`` where ``ydot_i``
    is the directional derivative of ``f_W(k_i)`` along the cotangent: with
    ``a = k W1``, ``b = k W3``, ``s = silu(a)``, ``h = s b``,
    ``adot = k D1``, ``bdot = k D3``, ``hdot = silu'(a) adot b + s bdot``,
    ``ydot = hdot W2 + h D2``.  Writing ``g = v W2^T`` and ``r = v D2^T``,
    ``phi_i / eta_i = sum_u hdot_u g_u + h_u r_u``, whose partial
    derivatives (derived by hand) give
      ``d/dv = eta ydot``, ``d/deta = <ydot, v>``,
      ``Pa = silu''(a) adot b g + silu'(a) (bdot g + b r)`` (w.r.t. ``a``),
      ``Pb = silu'(a) adot g + s r`` (``b``), ``Padot = silu'(a) b g``,
      ``Pbdot = s g``, ``Pg = hdot`` (w.r.t. ``g``);
      ``d/dk = eta (Pa W1^T + Pb W3^T + Padot D1^T + Pbdot D3^T)``,
      ``d/dW1 = K^T (eta Pa)``, ``d/dW3 = K^T (eta Pb)``,
      ``d/dW2 = (eta Pg)^T V``.
    Returns ``(dK, dV, deta, (dW1, dW3, dW2))``."""
    K, V, eta, W1, W3, W2, D1, D3, D2 = map(_f64, (K, V, eta, W1, W3, W2, D1, D3, D2))
    tr = lambda M: np.swapaxes(M, -1, -2)  # noqa: E731
    e = eta[..., None]
    a, b = K @ W1, K @ W3
    s, s1, s2 = silu(a), silu_prime(a), silu_second(a)
    h = s * b
    ad, bd = K @ D1, K @ D3
    hd = s1 * ad * b + s * bd
    g, r = V @ tr(W2), V @ tr(D2)
    yd = hd @ W2 + h @ D2
    Pa = s2 * ad * b * g + s1 * (bd * g + b * r)
    Pb = s1 * ad * g + s * r
    Pad = s1 * b * g
    Pbd = s * g
    dK = e * (Pa @ tr(W1) + Pb @ tr(W3) + Pad @ tr(D1) + Pbd @ tr(D3))
    dV = e * yd
    deta = np.sum(yd * V, axis=-1)
    return dK, dV, deta, (tr(K) @ (e * Pa), tr(K) @ (e * Pb), tr(e * hd) @ V)


def _normalize_backward(U, G):
    """Gradient through ``W = U / max(||U column||, 1e-12)`` per column, given
    the gradient ``G`` of ``W``: ``(G - w (w . G)) / n`` (``G / 1e-12`` at the
    floor, where the map is linear)."""
    n = np.sqrt(np.sum(U * U, axis=-2, keepdims=True))
    w = U / np.maximum(n, NORM_EPS)
    return np.where(n > NORM_EPS, (G - w * np.sum(w * G, axis=-2, keepdims=True)) / np.maximum(n, NORM_EPS),
                    G / NORM_EPS)


def large_chunk_swiglu_backward(Q, K, V, eta, W1, W3, W2, dO, dW_T, chunk, read_first=True, normalize=True,
                                update_w1w3=True):
    """Reverse-mode gradients of :func:`large_chunk_swiglu` (plain descent):
    given ``dO`` and ``dW_T = (dW1, dW3, dW2)`` of the final weights, return
    ``(dQ, dK, dV, deta, (dW1_0, dW3_0, dW2_0))``.

    Derived by hand from the chunk loop, walked backwards.  Chunk c forms
    ``U_c = W_{c-1} + S(W_{c-1})`` (``S`` the eta-weighted descent step, see
    :func:`swiglu_step_vjp`) and ``W_c`` = its column normalisation; its
    queries read ``R_c = W_{c-1}`` (``W_c`` when not ``read_first``).  With
    ``G`` the gradient of the newest weights (``dW_T`` at the end), for each
    chunk from the last: update-first read: ``dQ_c`` and ``G +=`` the read's
    weight gradient at ``W_c`` (:func:`swiglu_read_backward`);
    normalisation: ``dU = (G - w (w . G)) / n`` per column; step: the
    weights before it get ``dU`` plus the step's vector-Jacobian product with
    ``dU``, and ``dK_c``, ``dV_c``, ``deta_c`` come from the same product;
    read-first read: ``dQ_c`` and the read's weight gradient at ``W_{c-1}``.
    A matrix the loop does not update (``update_w1w3=False``) passes ``G`` on
    unchanged and gets only the step's product (through the hidden features).
    ``dW0`` is ``G`` after the first chunk."""
    Q, K, V, eta, dO = map(_f64, (Q, K, V, eta, dO))
    Ws = [tuple(_f64(w).copy() for w in (W1, W3, W2))]
    Us = []
    T = Q.shape[2]
    starts = list(range(0, T, chunk))
    upd = (update_w1w3, update_w1w3, True)
    for s0 in starts:
        e = min(s0 + chunk, T)
        g = swiglu_binding_grad(K[:, :, s0:e], V[:, :, s0:e], eta[:, :, s0:e], *Ws[-1])
        U = tuple(w - gg if u else w for w, gg, u in zip(Ws[-1], g, upd))
        Us.append(U)
        Ws.append(tuple(normalize_columns(x) if (normalize and u) else x for x, u in zip(U, upd)))
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    deta = np.zeros_like(eta)
    G = [_f64(x).copy() for x in dW_T]
    for c in range(len(starts) - 1, -1, -1):
        s0, e = starts[c], min(starts[c] + chunk, T)
        if not read_first:
            dq, gr = swiglu_read_backward(Q[:, :, s0:e], *Ws[c + 1], dO[:, :, s0:e])
            dQ[:, :, s0:e] = dq
            G = [x + y for x, y in zip(G, gr)]
        dU = [(_normalize_backward(u, x) if normalize else x) if up else np.zeros_like(x)
              for u, x, up in zip(Us[c], G, upd)]
        dk, dv, de, gs = swiglu_step_vjp(K[:, :, s0:e], V[:, :, s0:e], eta[:, :, s0:e], *Ws[c], *dU)
        dK[:, :, s0:e], dV[:, :, s0:e], deta[:, :, s0:e] = dk, dv, de
        G = [(d if up else x) + y for d, x, y, up in zip(dU, G, gs, upd)]
        if read_first:
            dq, gr = swiglu_read_backward(Q[:, :, s0:e], *Ws[c], dO[:, :, s0:e])
            dQ[:, :, s0:e] = dq
            G = [x + y for x, y in zip(G, gr)]
    return dQ, dK, dV, deta, tuple(G)


def backward(Q, K, V, eta, W0, dO, dW_T, chunk, mode, d_h=None):
    """Gradients ``(dQ, dK, dV, deta, dW0)`` by mode name, with the
    library's argument order.  For the SwiGLU modes ``W0`` and ``dW_T`` are
    packed states and ``d_h`` is required; ``dW0`` is returned packed."""
    if mode in ("per_token_linear", "per_token_linear_exclusive"):
        return per_token_linear_backward(Q, K, V, eta, W0, dO, dW_T, inclusive=(mode == "per_token_linear"))
    if mode in ("large_chunk_linear", "large_chunk_linear_update_first"):
        return large_chunk_linear_backward(Q, K, V, eta, W0, dO, dW_T, chunk,
                                           read_first=(mode == "large_chunk_linear"))
    if mode in ("large_chunk_swiglu", "large_chunk_swiglu_update_first", "large_chunk_swiglu_last_layer"):
        d = Q.shape[-1]
        last = mode == "large_chunk_swiglu_last_layer"
        dq, dk, dv, de, G = large_chunk_swiglu_backward(
            Q, K, V, eta, *swiglu_unpack(_f64(W0), d, d_h), dO, swiglu_unpack(_f64(dW_T), d, d_h), chunk,
            read_first=(mode != "large_chunk_swiglu_update_first"), normalize=not last, update_w1w3=not last)
        return dq, dk, dv, de, swiglu_pack(*G)
    raise ValueError(f"no backward for mode {mode!r}")


def large_chunk_linear(Q, K, V, eta, W0, chunk, normalize=True, read_first=True, momentum=None, M0=None):
    """LaCT with a linear fast weight.  For each chunk (the last may be
    shorter): every query of the chunk reads W (the state left by earlier
    chunks); then W takes one step on the chunk's summed, eta-weighted
    binding loss; then each output unit's fan-in is L2-normalised.

    LaCT review: fast-weights section (one update per large chunk),
    non-linear-memory section (summed per-token-rate gradients, L2
    normalisation after the update), read-order section (a chunk reads
    the memory of earlier chunks and only then updates it).
    ``read_first=False``: the chunk's queries read W after its update.
    ``normalize=False`` is an oracle-only switch used by the pins.
    ``momentum=beta`` (LaCT review, non-linear-memory section, which
    compares momentum in the inner loop): the step applied is a momentum
    buffer ``M_c = beta M_{c-1} - grad_c`` (``M`` starts at ``M0``, zeros
    by default), then the normalisation; returns (O, W, M) instead."""
    Q, K, V, eta, W = map(_f64, (Q, K, V, eta, W0))
    W = W.copy()
    M = np.zeros_like(W) if M0 is None else _f64(M0).copy()
    T = Q.shape[2]
    O = np.zeros(Q.shape[:-1] + (V.shape[-1],))
    for s in range(0, T, chunk):
        e = min(s + chunk, T)
        if read_first:
            O[:, :, s:e, :] = np.matmul(Q[:, :, s:e, :], W)
        g = linear_binding_grad(K[:, :, s:e, :], V[:, :, s:e, :], eta[:, :, s:e])
        if momentum is None:
            W = W - g
        else:
            M = momentum * M - g
            W = W + M
        if normalize:
            W = normalize_columns(W)
        if not read_first:
            O[:, :, s:e, :] = np.matmul(Q[:, :, s:e, :], W)
    if momentum is not None:
        return O, W, M
    return O, W


# Coefficients of the quintic Newton-Schulz iteration of the Muon optimizer
# (K. Jordan et al., "Muon: An optimizer for hidden layers in neural
# networks", 2024): each step maps every singular value s of the normalised
# matrix to a s + b s^3 + c s^5, which drives all of them towards a band
# around 1 in five steps.
NS_COEFFS = (3.4445, -4.7750, 2.0315)
NS_STEPS = 5
NS_EPS = 1e-7


def newton_schulz5(G):
    """Approximate orthogonalisation of a matrix step by the Muon iteration
    (LaCT review, non-linear memory section: Muon transforms the matrix
    gradients by Newton-Schulz iterations).  Over the last two axes:
    ``X = G / (||G||_F + 1e-7)``, transposed when it has more rows than
    columns; five times ``A = X X^T``, ``X = a X + (b A + c A A) X``; then
    transposed back.  With ``G = U diag(s) V^T`` the result is
    ``U diag(p(s / (||G||_F + 1e-7))) V^T``, ``p`` the scalar quintic
    applied five times."""
    a, b, c = NS_COEFFS
    X = _f64(G)
    X = X / (np.sqrt(np.sum(X * X, axis=(-2, -1), keepdims=True)) + NS_EPS)
    tall = X.shape[-2] > X.shape[-1]
    if tall:
        X = np.swapaxes(X, -1, -2)
    for _ in range(NS_STEPS):
        A = np.matmul(X, np.swapaxes(X, -1, -2))
        X = a * X + np.matmul(b * A + c * np.matmul(A, A), X)
    if tall:
        X = np.swapaxes(X, -1, -2)
    return X


def large_chunk_swiglu(Q, K, V, eta, W1, W3, W2, chunk, normalize=True,
                       update_w1w3=True, read_first=True, momentum=None, M0=None, muon_scale=None):
    """LaCT with a SwiGLU fast-weight MLP.  For each chunk: the chunk's
    queries read ``f_W``; the eta-weighted binding-loss gradient of the
    chunk is taken at those same weights; one descent step is applied to
    W1, W3, W2; then each output unit is L2-normalised (W1, W3 columns over
    d, W2 columns over d_h).

    LaCT review, non-linear memory and read-order sections.
    ``read_first=False``: the chunk's queries read the weights after its
    update (the gradient is still taken at the weights before it).
    ``normalize=False`` with ``update_w1w3=False`` is the last-layer-only
    variant of the paper summary's ablation ladder (technical section 4:
    train only the last layer, then drop the weight normalisation).

    Update rules the LaCT review's non-linear-memory section compares with
    plain descent: ``momentum=beta`` keeps one buffer per matrix,
    ``M = beta M + step`` (``step`` = minus the chunk's gradient; ``M``
    starts at ``M0 = (M1, M3, M2)``, zeros by default), and the weights take
    ``M`` instead of the step; ``muon_scale=s`` replaces what the weights
    take (the step, or ``M``) by ``s * newton_schulz5(.)`` of it, matrix by
    matrix.  The normalisation follows either.  Returns (O, (W1, W3, W2)),
    plus (M1, M3, M2) when ``momentum`` is given."""
    Q, K, V, eta, W1, W3, W2 = map(_f64, (Q, K, V, eta, W1, W3, W2))
    W1, W3, W2 = W1.copy(), W3.copy(), W2.copy()
    if M0 is None:
        M = [np.zeros_like(W1), np.zeros_like(W3), np.zeros_like(W2)]
    else:
        M = [_f64(m).copy() for m in M0]
    T = Q.shape[2]
    O = np.zeros(Q.shape[:-1] + (W2.shape[-1],))
    for s in range(0, T, chunk):
        e = min(s + chunk, T)
        if read_first:
            O[:, :, s:e, :] = swiglu_forward(Q[:, :, s:e, :], W1, W3, W2)
        g1, g3, g2 = swiglu_binding_grad(K[:, :, s:e, :], V[:, :, s:e, :],
                                         eta[:, :, s:e], W1, W3, W2)
        steps = [-g1, -g3, -g2]                # descent on the binding loss
        if momentum is not None:
            M = [momentum * m + st for m, st in zip(M, steps)]
            steps = list(M)
        if muon_scale is not None:
            steps = [muon_scale * newton_schulz5(st) for st in steps]
        if update_w1w3:
            W1 = W1 + steps[0]
            W3 = W3 + steps[1]
        W2 = W2 + steps[2]
        if normalize:
            if update_w1w3:
                W1 = normalize_columns(W1)
                W3 = normalize_columns(W3)
            W2 = normalize_columns(W2)
        if not read_first:
            O[:, :, s:e, :] = swiglu_forward(Q[:, :, s:e, :], W1, W3, W2)
    if momentum is not None:
        return O, (W1, W3, W2), tuple(M)
    return O, (W1, W3, W2)


# ---------------------------------------------------------------------------
# Packing helpers for the SwiGLU state buffer [B,H] x (W1 | W3 | W2)
# ---------------------------------------------------------------------------

def swiglu_pack(W1, W3, W2):
    """Concatenate per-head (W1 [d,d_h], W3 [d,d_h], W2 [d_h,d]) row-major
    into one ``[B,H,3*d*d_h]`` array (the state buffer layout)."""
    B, H = W1.shape[:2]
    return np.concatenate([W1.reshape(B, H, -1), W3.reshape(B, H, -1),
                           W2.reshape(B, H, -1)], axis=-1)


def swiglu_unpack(Wp, d, d_h):
    """Inverse of :func:`swiglu_pack`."""
    B, H = Wp.shape[:2]
    n = d * d_h
    return (Wp[..., :n].reshape(B, H, d, d_h), Wp[..., n:2 * n].reshape(B, H, d, d_h),
            Wp[..., 2 * n:].reshape(B, H, d_h, d))


def forward(Q, K, V, eta, W0, chunk, mode, d_h=None):
    """Dispatch by mode name, with the library's argument order.

    ``mode``: "per_token_linear", "large_chunk_linear" or
    "large_chunk_swiglu", and the ordering variants
    "per_token_linear_exclusive" (a query reads before its token's update),
    "large_chunk_linear_update_first" and "large_chunk_swiglu_update_first"
    (a chunk updates, then reads), and "large_chunk_swiglu_last_layer"
    (only W2 trained, no normalisation).  For per-token mode ``chunk`` does not
    change the result and is ignored.  For SwiGLU, W0 is the packed state and
    ``d_h`` is required.  Returns (O, W_final) with W_final in W0's layout."""
    if mode in ("per_token_linear", "per_token_linear_exclusive"):
        return per_token_linear(Q, K, V, eta, W0, inclusive=(mode == "per_token_linear"))
    if mode in ("large_chunk_linear", "large_chunk_linear_update_first"):
        return large_chunk_linear(Q, K, V, eta, W0, chunk, read_first=(mode == "large_chunk_linear"))
    if mode in ("large_chunk_swiglu", "large_chunk_swiglu_update_first"):
        d = Q.shape[-1]
        W1, W3, W2 = swiglu_unpack(_f64(W0), d, d_h)
        O, (W1, W3, W2) = large_chunk_swiglu(Q, K, V, eta, W1, W3, W2, chunk,
                                             read_first=(mode == "large_chunk_swiglu"))
        return O, swiglu_pack(W1, W3, W2)
    if mode == "large_chunk_swiglu_last_layer":
        d = Q.shape[-1]
        W1, W3, W2 = swiglu_unpack(_f64(W0), d, d_h)
        O, (W1, W3, W2) = large_chunk_swiglu(Q, K, V, eta, W1, W3, W2, chunk, normalize=False, update_w1w3=False)
        return O, swiglu_pack(W1, W3, W2)
    raise ValueError(f"unknown mode {mode!r}")
