"""Plain, slow fp64 CPU oracle of the large-chunk test-time-training (TTT) layer forward.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import or run this module. It shares no code with the HIP library: the two meet only
in the seeded input generator (``ttt_inputs``), which holds none of the layer's arithmetic.

Sources (cited by page and section; the pages' own equation text did not survive
extraction, so the formulas below are the plain forms the pages describe in words):

* [LaCT] "LaCT技术解析：大块测试时训练提升长序列建模效率" (peacm.com):
  §1.2 update once per large chunk of 2K-1M tokens; "key implementation tricks":
  a SwiGLU-MLP fast-weight net updated with Muon; §2.1 the TTT layer's two phases --
  update (the chunk's summed gradient moves the fast weights, eqs. 4-5) and apply (the
  fast weights are applied to every query of the chunk, eq. 2); §2.2.1 L2 weight
  normalisation of the fast weights (eq. 8) and Muon turning the gradient into an
  orthogonal matrix by approximate SVD (eqs. 9-10); §3.2 shifted block-causal mask
  (Fig. 3c) for text; §3.1 one whole-sequence chunk for image sets.
* [TTT layers] "Что такое Test-Time Training (TTT) слои" (aivaro.ru): §3 the per-step
  recurrence theta_t = theta_{t-1} - eta * grad L, output h_t = f_theta(x_t), an MSE
  self-supervised loss; §4 a 2-layer MLP inner model trained by SGD; §10 the scalar
  sine-wave exercise (d = 1, y = w*x, MSE on the previous token, lr 0.01).
* [Modular TTT] arxivdaily.com abstract "Modular TTT": MSE and inner-product inner
  losses as interchangeable design dimensions.
* [TTT-E2E] "TTT-E2E端到端测试时训练方法解析" (jsqmd.com): §2.1.2 delta rule -- a weight
  change is an outer product of the back-propagated error (times the activation
  derivative) with the layer input.

Readings where the pages are silent (each one is listed in the design notes):
* loss of a chunk S: inner product  L = -sum_{t in S} eta_t <f_W(k_t), v_t>,  or
  MSE  L = sum_{t in S} eta_t ||f_W(k_t) - v_t||^2  (no 1/2, no 1/d, no 1/|S|);
* one eta per token, shared by all fast-weight matrices; momentum off unless the config
  sets it (heavy-ball over chunks, momentum_step); the update is
  W <- (1 - lambda) W - lr_i U with U the gradient (SGD) or its 5-step Newton-Schulz
  orthogonalisation (Muon), lr_i a step size per matrix (default 1: the step the pages
  describe) and lambda a weight decay (default 0) -- [Modular TTT] names the learning
  rate and the weight decay as design dimensions of the inner learner, and [LaCT] §4.2
  suggests a smaller Muon step when the loss oscillates; the decay scales the state
  before the step, and the row renorm's reference is the norm before decay and step;
* Newton-Schulz: X = G / (||G||_F + 1e-7), transposed to the wide orientation,
  5 x { A = X X^T ; B = b A + c A^2 ; X = a X + B X } with the quintic coefficients
  (a, b, c) = (3.4445, -4.7750, 2.0315) published with the Muon optimiser;
* row renorm: after W' = (1 - lambda) W - lr U every row of every matrix is rescaled to
  the L2 norm that row had before the update; a row whose new norm is 0 is left as it is;
* shifted block-causal: chunk c's queries see the state after chunks 0..c-1 and the
  last chunk's update is still made; the image-set order updates first, then applies;
* SwiGLU  f(x) = W2 (silu(W1 x) * (W3 x));  GELU-MLP  f(x) = W2 gelu(W1 x) with the
  exact erf GELU; no biases, no norms, no residual inside f.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np
from scipy.special import erf

MUON_COEFFS = (3.4445, -4.7750, 2.0315)
NS_EPS = 1e-7

APPLY_THEN_UPDATE = "apply_then_update"
UPDATE_THEN_APPLY = "update_then_apply"


# ----------------------------------------------------------------------------- activations
def sigmoid(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    return z * sigmoid(z)


def silu_prime(z):
    # d/dz [z s(z)] = s + z s (1 - s)
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def gelu(z):
    return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


def gelu_prime(z):
    # d/dz [z Phi(z)] = Phi(z) + z phi(z)
    return 0.5 * (1.0 + erf(z / np.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)


# ------------------------------------------------------------------------- fast-weight net
def fw_apply(fw: str, Ws: Sequence[np.ndarray], X: np.ndarray) -> np.ndarray:
    """f_W applied to every row of X (rows are tokens). [LaCT] §2.1 apply phase (eq. 2);
    SwiGLU net per [LaCT] "key implementation tricks"; GELU MLP per [TTT layers] §4."""
    X = np.asarray(X, dtype=np.float64)
    if fw == "swiglu":
        W1, W3, W2 = Ws
        return (silu(X @ W1.T) * (X @ W3.T)) @ W2.T
    if fw == "gelu":
        W1, W2 = Ws
        return gelu(X @ W1.T) @ W2.T
    if fw == "linear":
        (W,) = Ws
        return X @ W.T
    raise ValueError(fw)


def chunk_loss(fw: str, loss: str, Ws, K, V, eta) -> float:
    """Value of the chunk's inner loss (used by the finite-difference pins)."""
    F = fw_apply(fw, Ws, K)
    V = np.asarray(V, np.float64)
    eta = np.asarray(eta, np.float64)
    if loss == "dot":
        return float(-np.sum(eta * np.sum(F * V, axis=1)))
    if loss == "mse":
        return float(np.sum(eta * np.sum((F - V) ** 2, axis=1)))
    raise ValueError(loss)


def _output_error(loss: str, F_k: Optional[np.ndarray], V: np.ndarray, eta: np.ndarray):
    """dL/df(k_t) per token: -eta v (inner product) or 2 eta (f(k) - v) (MSE)."""
    if loss == "dot":
        return -eta[:, None] * V
    if loss == "mse":
        return 2.0 * eta[:, None] * (F_k - V)
    raise ValueError(loss)


def _block_gradient(fw: str, loss: str, Ws, K, V, eta) -> List[np.ndarray]:
    """Gradient of the loss over one block of tokens, matrix form (token sums are
    matrix products). Chain rule through the net; the weight gradients are the
    token-summed outer products of back-propagated errors with layer inputs
    ([TTT-E2E] §2.1.2)."""
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    eta = np.asarray(eta, np.float64)
    if fw == "swiglu":
        W1, W3, W2 = Ws
        Z1 = K @ W1.T
        Z3 = K @ W3.T
        A = silu(Z1)
        H = A * Z3
        E = _output_error(loss, H @ W2.T if loss == "mse" else None, V, eta)
        g2 = E.T @ H
        dH = E @ W2
        dZ3 = dH * A
        dZ1 = dH * Z3 * silu_prime(Z1)
        return [dZ1.T @ K, dZ3.T @ K, g2]
    if fw == "gelu":
        W1, W2 = Ws
        Z = K @ W1.T
        H = gelu(Z)
        E = _output_error(loss, H @ W2.T if loss == "mse" else None, V, eta)
        g2 = E.T @ H
        dZ = (E @ W2) * gelu_prime(Z)
        return [dZ.T @ K, g2]
    if fw == "linear":
        (W,) = Ws
        E = _output_error(loss, K @ W.T if loss == "mse" else None, V, eta)
        return [E.T @ K]
    raise ValueError(fw)


def apply_vjp(fw: str, Ws, Q, dO):
    """Backward of one chunk's apply step O = f_W(Q) ([LaCT] §2.1 apply phase; the
    query-view rule that [Modular TTT] composes into the layer's backward): given dO, the
    gradients of sum_t <dO_t, f_W(q_t)> with respect to Q and to every matrix of W, by the
    chain rule through the net. Returns (dQ [n, d], [dW per matrix])."""
    Q = np.asarray(Q, np.float64)
    dO = np.asarray(dO, np.float64)
    if fw == "swiglu":
        W1, W3, W2 = Ws
        Z1 = Q @ W1.T
        Z3 = Q @ W3.T
        A = silu(Z1)
        H = A * Z3
        dH = dO @ W2
        dZ3 = dH * A
        dZ1 = dH * Z3 * silu_prime(Z1)
        return dZ1 @ W1 + dZ3 @ W3, [dZ1.T @ Q, dZ3.T @ Q, dO.T @ H]
    if fw == "gelu":
        W1, W2 = Ws
        Z = Q @ W1.T
        dZ = (dO @ W2) * gelu_prime(Z)
        return dZ @ W1, [dZ.T @ Q, dO.T @ gelu(Z)]
    if fw == "linear":
        (W,) = Ws
        return dO @ W, [dO.T @ Q]
    raise ValueError(fw)


def chunk_gradient(fw: str, loss: str, Ws, K, V, eta, block_rows: Optional[int] = None):
    """Sum of the per-token gradients over the whole chunk ([LaCT] §2.1 update phase,
    eqs. 4-5). A chunk longer than ``block_rows`` is summed block by block: the
    gradient of a sum of per-token losses is the sum of the blocks' gradients."""
    n = len(eta)
    if block_rows is None or n <= block_rows:
        return _block_gradient(fw, loss, Ws, K, V, eta)
    total = None
    for s in range(0, n, block_rows):
        g = _block_gradient(fw, loss, Ws, K[s:s + block_rows], V[s:s + block_rows],
                            eta[s:s + block_rows])
        total = g if total is None else [t + x for t, x in zip(total, g)]
    return total


# ----------------------------------------------------------------- optimiser and weight norm
def newton_schulz5(G: np.ndarray, steps: int = 5, coeffs=MUON_COEFFS, eps: float = NS_EPS):
    """Muon's orthogonalisation of a gradient matrix ([LaCT] §2.2.1, eqs. 9-10): scale
    to unit Frobenius norm, then ``steps`` quintic Newton-Schulz iterations, run in the
    wide orientation (rows <= cols) and transposed back."""
    a, b, c = coeffs
    X = np.asarray(G, np.float64) / (np.linalg.norm(G) + eps)
    wide = X.shape[0] <= X.shape[1]
    if not wide:
        X = X.T
    for _ in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X if wide else X.T


def renorm_rows(W_prev: np.ndarray, W_new: np.ndarray) -> np.ndarray:
    """L2 weight normalisation ([LaCT] §2.2.1, eq. 8): each row of the updated matrix
    is rescaled to the L2 norm the same row had before the update."""
    n_prev = np.linalg.norm(W_prev, axis=1)
    n_new = np.linalg.norm(W_new, axis=1)
    ok = n_new > 0
    scale = np.where(ok, n_prev / np.where(ok, n_new, 1.0), 1.0)
    return W_new * scale[:, None]


def update_state(Ws, grads, ns_steps: int, renorm: bool, lr: Optional[Sequence[float]] = None,
                 weight_decay: float = 0.0) -> List[np.ndarray]:
    """W <- (1 - weight_decay) W - lr_i U per matrix, U = NS5(g) under Muon else g
    ([LaCT] §2.2.1; step size and weight decay as in [Modular TTT]); then the optional
    row renorm against the norms of W before this update."""
    out = []
    steps = [1.0] * len(Ws) if lr is None else list(lr)
    for W, g, step in zip(Ws, grads, steps):
        U = newton_schulz5(g, ns_steps) if ns_steps > 0 else g
        W_new = (1.0 - weight_decay) * W - step * U
        out.append(renorm_rows(W, W_new) if renorm else W_new)
    return out


def momentum_step(Ms, grads, beta: float):
    """Heavy-ball accumulation of the chunk gradients, M <- beta M + g per matrix: the
    ordinary momentum optimiser that [LaCT] §2.2.1 compares its Muon variant with; under
    Muon the orthogonalisation is applied to M, as the published Muon optimiser does with
    its momentum buffer."""
    return [beta * np.asarray(M, np.float64) + g for M, g in zip(Ms, grads)]


# ------------------------------------------------------------------------- the layer loop
def sequence_forward(cfg, W0s, Q, K, V, eta, block_rows: Optional[int] = 8192,
                     apply_rows: Optional[np.ndarray] = None, n_chunks: Optional[int] = None,
                     update_chunks: Optional[Sequence[bool]] = None):
    """One (batch, head) problem: the chunk loop of the TTT layer.

    W0s: the problem's initial matrices; Q, K, V: [T, d]; eta: [T].
    Chunk c covers tokens [c*b, (c+1)*b). Under the shifted block-causal order
    ([LaCT] §3.2, Fig. 3c) its queries are answered with the state left by chunks
    0..c-1 and its own update follows; the image-set order ([LaCT] §3.1) updates
    first and then applies. The state after the last chunk is returned.

    update_chunks: optional flag per chunk; a chunk whose flag is false answers its
    queries with the state as it stands and leaves the state unchanged (no gradient, no
    decay, no renorm): the fast weights are updated on chosen chunks only, as [LaCT] §3.3
    does for the clean-frame chunks of an autoregressive video sequence.
    apply_rows: optional sorted token indices; only those rows of O are computed
    (the others stay 0). n_chunks: stop after that many chunks.
    With cfg.momentum = beta > 0 the chunk gradients pass through momentum_step (the
    buffers start at zero) and the returned matrices are the fast weights followed by the
    momentum buffers.
    Returns (O [T, d] fp64, list of final fp64 matrices)."""
    T = len(eta)
    b = cfg.chunk
    Ws = [np.asarray(w, np.float64) for w in W0s]
    beta = float(getattr(cfg, "momentum", 0.0))
    Ms = [np.zeros_like(w) for w in Ws] if beta else None
    O = np.zeros((T, cfg.dim), np.float64)
    nc = T // b if n_chunks is None else n_chunks
    rows = None if apply_rows is None else np.asarray(apply_rows)

    def apply(lo, hi):
        if rows is None:
            for s in range(lo, hi, block_rows or (hi - lo)):
                e = min(hi, s + (block_rows or (hi - lo)))
                O[s:e] = fw_apply(cfg.fw, Ws, Q[s:e])
        else:
            sel = rows[(rows >= lo) & (rows < hi)]
            if len(sel):
                O[sel] = fw_apply(cfg.fw, Ws, Q[sel])

    for c in range(nc):
        lo, hi = c * b, (c + 1) * b
        if update_chunks is not None and not update_chunks[c]:
            apply(lo, hi)
            continue
        if cfg.order == APPLY_THEN_UPDATE:
            apply(lo, hi)
        g = chunk_gradient(cfg.fw, cfg.loss, Ws, K[lo:hi], V[lo:hi], eta[lo:hi], block_rows)
        if Ms is not None:
            Ms = momentum_step(Ms, g, beta)
            g = Ms
        Ws = update_state(Ws, g, cfg.ns_steps, cfg.renorm, cfg.step_sizes(), cfg.weight_decay)
        if cfg.order == UPDATE_THEN_APPLY:
            apply(lo, hi)
    return O, (Ws + Ms if Ms is not None else Ws)


def sequence_forward_bruteforce(cfg, W0s, Q, K, V, eta, update_chunks=None):
    """Per-token version for tiny inputs: every output row and every token's gradient
    is formed with explicit vector operations in Python loops, and the chunk gradient
    is the running sum of per-token outer products. Checks the matrix form above."""
    T = len(eta)
    b = cfg.chunk
    Ws = [np.array(w, np.float64) for w in W0s]
    O = np.zeros((T, cfg.dim))
    beta = float(getattr(cfg, "momentum", 0.0))
    Ms = [np.zeros_like(w) for w in Ws]

    def f(x):
        if cfg.fw == "swiglu":
            W1, W3, W2 = Ws
            z1, z3 = W1 @ x, W3 @ x
            return W2 @ (silu(z1) * z3)
        if cfg.fw == "gelu":
            W1, W2 = Ws
            return W2 @ gelu(W1 @ x)
        (W,) = Ws
        return W @ x

    for c in range(T // b):
        updates = update_chunks is None or bool(update_chunks[c])
        if cfg.order == APPLY_THEN_UPDATE or not updates:
            for t in range(c * b, (c + 1) * b):
                O[t] = f(np.asarray(Q[t], np.float64))
        if not updates:
            continue
        grads = [np.zeros_like(w) for w in Ws]
        for t in range(c * b, (c + 1) * b):
            k = np.asarray(K[t], np.float64)
            v = np.asarray(V[t], np.float64)
            et = float(eta[t])
            e = -et * v if cfg.loss == "dot" else 2.0 * et * (f(k) - v)
            if cfg.fw == "swiglu":
                W1, W3, W2 = Ws
                z1, z3 = W1 @ k, W3 @ k
                h = silu(z1) * z3
                dh = W2.T @ e
                grads[2] += np.outer(e, h)
                grads[0] += np.outer(dh * z3 * silu_prime(z1), k)
                grads[1] += np.outer(dh * silu(z1), k)
            elif cfg.fw == "gelu":
                W1, W2 = Ws
                z = W1 @ k
                grads[1] += np.outer(e, gelu(z))
                grads[0] += np.outer((W2.T @ e) * gelu_prime(z), k)
            else:
                grads[0] += np.outer(e, k)
        if beta:
            for i in range(len(Ms)):          # the momentum buffer, entry by entry
                for idx in np.ndindex(Ms[i].shape):
                    Ms[i][idx] = beta * Ms[i][idx] + grads[i][idx]
            grads = [M.copy() for M in Ms]
        Ws = update_state(Ws, grads, cfg.ns_steps, cfg.renorm, cfg.step_sizes(),
                          cfg.weight_decay)
        if cfg.order == UPDATE_THEN_APPLY:
            for t in range(c * b, (c + 1) * b):
                O[t] = f(np.asarray(Q[t], np.float64))
    return O, (Ws + Ms if beta else Ws)


def forward_all(cfg, inputs, problems: Optional[Sequence[Tuple[int, int]]] = None,
                block_rows: Optional[int] = 8192, update_chunks=None):
    """Run every (batch, head) problem (or the listed ones) of an input set made by
    ``ttt_inputs.make_inputs``. Returns {(b, h): (O, [W...])}."""
    out = {}
    probs = problems if problems is not None else [
        (b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    for (b, h) in probs:
        W0s = [w[h] for w in inputs["w0"]]
        out[(b, h)] = sequence_forward(cfg, W0s, inputs["q"][b, h], inputs["k"][b, h],
                                       inputs["v"][b, h], inputs["eta"][b, h], block_rows,
                                       update_chunks=update_chunks)
    return out


# ---------------------------------------------------------- backward through one chunk's update
# The outer loop of [E2E-2] §2.2 trains through the inner updates: the gradient of an outer
# loss reaches the inputs and the initial fast weights through every chunk's apply and update
# (the second-order gradients [E2E-2] §5.1 names as the cost of meta-learning); [Modular TTT]
# composes the layer's backward from the train view's forward and backward. These functions
# take one chunk's step backward with the chain rule, step by step in the forward's order.

def silu_second(z):
    # d/dz [s (1 + z (1 - s))] = s (1 - s) (2 + z (1 - 2 s))
    s = sigmoid(z)
    return s * (1.0 - s) * (2.0 + z * (1.0 - 2.0 * s))


def gelu_second(z):
    # d/dz [Phi(z) + z phi(z)] = phi(z) (2 - z^2)
    return np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi) * (2.0 - z * z)


def gradient_vjp(fw: str, loss: str, Ws, K, V, eta, dG):
    """Backward of the chunk gradient g(W, K, V, eta) = grad_W L (the update phase of [LaCT]
    §2.1) for a cotangent dG (one array per matrix, shaped like W): the gradients of
    phi = sum_m <dG_m, g_m> with respect to W, K, V and eta. phi is the derivative of L
    along the weight direction dG, so with J_t the forward-mode tangent of f_W(k_t) along dG
    and e_t = dL/df(k_t) the per-token output error, phi = sum_t <e_t, J_t>; its gradients
    follow by the chain rule through J_t (second derivatives of the activation) and, for the
    MSE loss, through e_t. Returns ([dW per matrix], dK, dV, deta)."""
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    eta = np.asarray(eta, np.float64)
    dG = [np.asarray(x, np.float64) for x in dG]
    if fw == "swiglu":
        W1, W3, W2 = Ws
        D1, D3, D2 = dG
        Z1, Z3 = K @ W1.T, K @ W3.T
        S, S1, S2 = silu(Z1), silu_prime(Z1), silu_second(Z1)
        H = S * Z3
        F = H @ W2.T
        E = _output_error(loss, F, V, eta)
        Dl = E @ W2                                  # hidden error, per token W2^T e_t
        Zd1, Zd3 = K @ D1.T, K @ D3.T                # tangents of Z1, Z3 along dG
        Hd = S1 * Zd1 * Z3 + S * Zd3                 # tangent of H
        J = H @ D2.T + Hd @ W2.T                     # tangent of f(k_t)
        G2 = E @ D2                                  # per token D2^T e_t
        dZ1, dZ3 = Dl * S1 * Z3, Dl * S              # the forward's back-propagated errors
        A1 = G2 * S1 * Z3 + Dl * (S2 * Zd1 * Z3 + S1 * Zd3)   # d phi / d Z1
        A3 = G2 * S + Dl * S1 * Zd1                           # d phi / d Z3
        dW = [A1.T @ K, A3.T @ K, E.T @ Hd]
        dK = A1 @ W1 + A3 @ W3 + dZ1 @ D1 + dZ3 @ D3
    elif fw == "gelu":
        W1, W2 = Ws
        D1, D2 = dG
        Z = K @ W1.T
        H, G1, Gs = gelu(Z), gelu_prime(Z), gelu_second(Z)
        F = H @ W2.T
        E = _output_error(loss, F, V, eta)
        Dl = E @ W2
        Zd = K @ D1.T
        Hd = G1 * Zd
        J = H @ D2.T + Hd @ W2.T
        G2 = E @ D2
        A1 = G2 * G1 + Dl * Gs * Zd
        dW = [A1.T @ K, E.T @ Hd]
        dK = A1 @ W1 + (Dl * G1) @ D1
    elif fw == "linear":
        (W,) = Ws
        (D,) = dG
        F = K @ W.T
        E = _output_error(loss, F, V, eta)
        J = K @ D.T
        dW = [np.zeros_like(W)]
        dK = E @ D
    else:
        raise ValueError(fw)
    if loss == "dot":                                # e_t = -eta_t v_t
        dV = -eta[:, None] * J
        deta = -np.sum(V * J, axis=1)
    elif loss == "mse":                              # e_t = 2 eta_t (f(k_t) - v_t)
        C = 2.0 * eta[:, None] * J                   # cotangent reaching f(k_t) through e_t
        dKf, dWf = apply_vjp(fw, Ws, K, C)
        dK = dK + dKf
        dW = [a + b for a, b in zip(dW, dWf)]
        dV = -C
        deta = 2.0 * np.sum((F - V) * J, axis=1)
    else:
        raise ValueError(loss)
    return dW, dK, dV, deta


def newton_schulz5_vjp(G: np.ndarray, dU: np.ndarray, steps: int = 5, coeffs=MUON_COEFFS,
                       eps: float = NS_EPS) -> np.ndarray:
    """Backward of newton_schulz5 ([LaCT] §2.2.1, eqs. 9-10) for a cotangent dU on its
    output: the iterates are recomputed, then each step X' = a X + (b A + c A A) X with
    A = X X^T is taken back (B symmetric), and finally the Frobenius scaling and the
    transposition to the wide orientation."""
    a, b, c = coeffs
    G = np.asarray(G, np.float64)
    nrm = np.linalg.norm(G)
    X = G / (nrm + eps)
    dX = np.asarray(dU, np.float64)
    wide = X.shape[0] <= X.shape[1]
    if not wide:
        X, dX = X.T, dX.T
    iterates = []
    for _ in range(steps):
        iterates.append(X)
        A = X @ X.T
        X = a * X + (b * A + c * (A @ A)) @ X
    for X in reversed(iterates):
        A = X @ X.T
        B = b * A + c * (A @ A)
        dB = dX @ X.T                               # X' = a X + B X
        dA = b * dB + c * (dB @ A + A @ dB)         # B = b A + c A A
        dX = a * dX + B.T @ dX + (dA + dA.T) @ X    # A = X X^T
    if not wide:
        dX = dX.T
    # X0 = G / (|G|_F + eps)
    if nrm == 0.0:
        return dX / eps
    return dX / (nrm + eps) - G * (np.sum(G * dX) / (nrm * (nrm + eps) ** 2))


def renorm_rows_vjp(W_prev: np.ndarray, W_new: np.ndarray, dOut: np.ndarray):
    """Backward of renorm_rows ([LaCT] §2.2.1, eq. 8): out_r = y_r |w_r| / |y_r| with
    y = W_new, w = W_prev (rows of zero new norm passed through). Returns (dW_prev, dW_new):
    the cotangent of y loses its component along y and is scaled by |w_r| / |y_r|; the
    reference norm |w_r| sends <y_r / |y_r|, dout_r> w_r / |w_r| to w_r."""
    W_prev = np.asarray(W_prev, np.float64)
    Y = np.asarray(W_new, np.float64)
    dOut = np.asarray(dOut, np.float64)
    n_prev = np.linalg.norm(W_prev, axis=1)
    n_new = np.linalg.norm(Y, axis=1)
    ok = n_new > 0
    yh = Y / np.where(ok, n_new, 1.0)[:, None]
    proj = np.sum(yh * dOut, axis=1)
    dY = np.where(ok[:, None], (n_prev / np.where(ok, n_new, 1.0))[:, None]
                  * (dOut - yh * proj[:, None]), dOut)
    scale_w = np.where(ok & (n_prev > 0), proj / np.where(n_prev > 0, n_prev, 1.0), 0.0)
    dW_prev = W_prev * scale_w[:, None]
    return dW_prev, dY


def update_state_vjp(Ws, grads, dWs_new, ns_steps: int, renorm: bool,
                     lr: Optional[Sequence[float]] = None, weight_decay: float = 0.0):
    """Backward of update_state for cotangents on the new matrices: returns (dW on the
    matrices before the update, dG on the chunk gradients)."""
    steps = [1.0] * len(Ws) if lr is None else list(lr)
    dW_out, dG_out = [], []
    for W, g, dWn, step in zip(Ws, grads, dWs_new, steps):
        W = np.asarray(W, np.float64)
        U = newton_schulz5(g, ns_steps) if ns_steps > 0 else np.asarray(g, np.float64)
        Y = (1.0 - weight_decay) * W - step * U
        if renorm:
            dW, dY = renorm_rows_vjp(W, Y, dWn)
        else:
            dW, dY = np.zeros_like(W), np.asarray(dWn, np.float64)
        dW = dW + (1.0 - weight_decay) * dY
        dU = -step * dY
        dG_out.append(newton_schulz5_vjp(g, dU, ns_steps) if ns_steps > 0 else dU)
        dW_out.append(dW)
    return dW_out, dG_out


def _split_momentum(cfg, Ws):
    """(matrices, momentum buffers, beta) of a state list: with cfg.momentum = beta > 0 the
    list holds the matrices followed by their buffers, else the matrices alone."""
    beta = float(getattr(cfg, "momentum", 0.0))
    nm = len(Ws) // 2 if beta else len(Ws)
    return list(Ws[:nm]), list(Ws[nm:]), beta


def chunk_step(cfg, Ws, Q, K, V, eta, update: bool = True):
    """One chunk of the layer loop (sequence_forward's body): (O, new state). With momentum
    the state is the matrices followed by their momentum buffers."""
    Ws = [np.asarray(w, np.float64) for w in Ws]
    W, M, beta = _split_momentum(cfg, Ws)
    if not update:
        return fw_apply(cfg.fw, W, Q), Ws
    O = fw_apply(cfg.fw, W, Q) if cfg.order == APPLY_THEN_UPDATE else None
    g = chunk_gradient(cfg.fw, cfg.loss, W, K, V, eta)
    if beta:
        M = momentum_step(M, g, beta)
        g = M
    Wn = update_state(W, g, cfg.ns_steps, cfg.renorm, cfg.step_sizes(), cfg.weight_decay)
    if O is None:
        O = fw_apply(cfg.fw, Wn, Q)
    return O, Wn + M


def chunk_vjp(cfg, Ws, Q, K, V, eta, dO, dWs_new, update: bool = True):
    """Backward of chunk_step: given the cotangents dO of the chunk's outputs and dWs_new of
    the state after it, the gradients of <dO, O> + sum_m <dW_new_m, W_new_m> with respect
    to the chunk's inputs and the state before it. The apply's part comes from apply_vjp
    (with the state the queries saw: before the update under the shifted order, after it
    under the update-then-apply order), the update's from update_state_vjp and
    gradient_vjp. With momentum the step's input is the new buffer M' = beta M + g: the
    cotangent of M' (from the step, plus the one given for the buffer after the chunk)
    reaches the chunk gradient whole and the buffer before the chunk times beta.
    Returns (dQ, dK, dV, deta, [dW before the chunk]) in the state's layout."""
    Ws = [np.asarray(w, np.float64) for w in Ws]
    dWs_new = [np.asarray(x, np.float64) for x in dWs_new]
    W, M, beta = _split_momentum(cfg, Ws)
    dWn, dMn, _ = _split_momentum(cfg, dWs_new)
    n = len(eta)
    if not update:
        dQ, dWa = apply_vjp(cfg.fw, W, Q, dO)
        return (dQ, np.zeros((n, cfg.dim)), np.zeros((n, cfg.dim)), np.zeros(n),
                [a + b for a, b in zip(dWn, dWa)] + dMn)
    g = chunk_gradient(cfg.fw, cfg.loss, W, K, V, eta)
    if beta:
        g = momentum_step(M, g, beta)
    if cfg.order == APPLY_THEN_UPDATE:
        dQ, dW_apply = apply_vjp(cfg.fw, W, Q, dO)
        dW_into_new = dWn
    else:
        Wn = update_state(W, g, cfg.ns_steps, cfg.renorm, cfg.step_sizes(), cfg.weight_decay)
        dQ, dWa_new = apply_vjp(cfg.fw, Wn, Q, dO)
        dW_apply = [np.zeros_like(w) for w in W]
        dW_into_new = [a + b for a, b in zip(dWn, dWa_new)]
    dW_step, dG = update_state_vjp(W, g, dW_into_new, cfg.ns_steps, cfg.renorm,
                                   cfg.step_sizes(), cfg.weight_decay)
    dM = []
    if beta:
        dG = [a + b for a, b in zip(dG, dMn)]
        dM = [beta * x for x in dG]
    dW_grad, dK, dV, deta = gradient_vjp(cfg.fw, cfg.loss, W, K, V, eta, dG)
    dW = [a + b + c for a, b, c in zip(dW_apply, dW_step, dW_grad)]
    return dQ, dK, dV, deta, dW + dM


def sequence_vjp(cfg, W0s, Q, K, V, eta, dO, dW_final=None, update_chunks=None):
    """Backward of sequence_forward for one problem: the states before every chunk are
    recomputed forward, then the chunks are taken back from the last to the first. With
    momentum the buffers start at zero, dW_final covers the matrices and then the buffers,
    and so does the returned list.
    Returns (dQ, dK, dV, deta, [dW0])."""
    T = len(eta)
    b = cfg.chunk
    Ws = [np.asarray(w, np.float64) for w in W0s]
    if getattr(cfg, "momentum", 0.0):
        Ws = Ws + [np.zeros_like(w) for w in Ws]
    states = []
    for c in range(T // b):
        states.append(Ws)
        S = slice(c * b, (c + 1) * b)
        up = update_chunks is None or bool(update_chunks[c])
        _, Ws = chunk_step(cfg, Ws, Q[S], K[S], V[S], eta[S], up)
    dW = [np.zeros_like(w) for w in Ws] if dW_final is None else \
        [np.asarray(x, np.float64) for x in dW_final]
    dQ, dK, dV = np.zeros((T, cfg.dim)), np.zeros((T, cfg.dim)), np.zeros((T, cfg.dim))
    deta = np.zeros(T)
    for c in reversed(range(T // b)):
        S = slice(c * b, (c + 1) * b)
        up = update_chunks is None or bool(update_chunks[c])
        dQ[S], dK[S], dV[S], deta[S], dW = chunk_vjp(cfg, states[c], Q[S], K[S], V[S], eta[S],
                                                     dO[S], dW, up)
    return dQ, dK, dV, deta, dW
