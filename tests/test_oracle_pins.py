"""Pins of the fp64 oracle to facts fixed outside the oracle itself.

Each pin compares the oracle with an independent route to the same number:
finite differences of the loss, torch autograd, per-token brute force, closed forms
of the linear fast weight, the scalar exercise of the TTT-layer explainer page, the
spectral form of the Newton-Schulz map, and invariants (eta = 0, row norms, causality).
The mutation tests at the end plant plausible mistakes in the oracle (on the CPU) and
check that some pin catches each one.
"""
import math

import numpy as np
import pytest
import torch

import oracle.ttt_oracle as orc
from ttt_inputs import Config

RNG = np.random.default_rng(12345)


def _rand_ws(fw, d, dh, rng, scale=0.5):
    shapes = {"swiglu": [(dh, d), (dh, d), (d, dh)], "gelu": [(dh, d), (d, dh)],
              "linear": [(d, d)]}[fw]
    return [rng.standard_normal(s) * scale for s in shapes]


def _rand_chunk(n, d, rng):
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    eta = 0.01 + 0.1 * rng.random(n)
    return K, V, eta


# ------------------------------------------------------------------ gradient pins
def fd_gradient_error(fw, loss, seed=0, d=4, dh=8, n=3, eps=1e-6):
    rng = np.random.default_rng(seed)
    Ws = _rand_ws(fw, d, dh, rng)
    K, V, eta = _rand_chunk(n, d, rng)
    g = orc.chunk_gradient(fw, loss, Ws, K, V, eta)
    worst = 0.0
    for i, W in enumerate(Ws):
        fd = np.zeros_like(W)
        for idx in np.ndindex(W.shape):
            Wp = [w.copy() for w in Ws]
            Wm = [w.copy() for w in Ws]
            Wp[i][idx] += eps
            Wm[i][idx] -= eps
            fd[idx] = (orc.chunk_loss(fw, loss, Wp, K, V, eta)
                       - orc.chunk_loss(fw, loss, Wm, K, V, eta)) / (2 * eps)
        worst = max(worst, np.abs(fd - g[i]).max() / np.abs(fd).max())
    return worst


@pytest.mark.parametrize("fw", ["swiglu", "gelu", "linear"])
@pytest.mark.parametrize("loss", ["dot", "mse"])
def test_gradient_matches_finite_differences(fw, loss):
    assert fd_gradient_error(fw, loss) < 1e-6


def _torch_loss(fw, loss, Ws, K, V, eta):
    F = torch.nn.functional
    if fw == "swiglu":
        W1, W3, W2 = Ws
        out = (F.silu(K @ W1.T) * (K @ W3.T)) @ W2.T
    elif fw == "gelu":
        W1, W2 = Ws
        out = F.gelu(K @ W1.T) @ W2.T
    else:
        (W,) = Ws
        out = K @ W.T
    if loss == "dot":
        return -(eta * (out * V).sum(1)).sum()
    return (eta * ((out - V) ** 2).sum(1)).sum()


@pytest.mark.parametrize("fw", ["swiglu", "gelu", "linear"])
@pytest.mark.parametrize("loss", ["dot", "mse"])
def test_gradient_matches_torch_autograd(fw, loss):
    rng = np.random.default_rng(7)
    Ws = _rand_ws(fw, 6, 10, rng)
    K, V, eta = _rand_chunk(5, 6, rng)
    g = orc.chunk_gradient(fw, loss, Ws, K, V, eta)
    tW = [torch.tensor(w, dtype=torch.float64, requires_grad=True) for w in Ws]
    L = _torch_loss(fw, loss, tW, torch.tensor(K), torch.tensor(V), torch.tensor(eta))
    tg = torch.autograd.grad(L, tW)
    for a, b in zip(g, tg):
        assert np.abs(a - b.numpy()).max() <= 1e-12 * max(1.0, np.abs(a).max())


def test_activations_match_torch():
    z = np.linspace(-8, 8, 1001)
    tz = torch.tensor(z, requires_grad=True)
    F = torch.nn.functional
    for ours, ours_d, theirs in ((orc.silu, orc.silu_prime, F.silu),
                                 (orc.gelu, orc.gelu_prime, F.gelu)):
        y = theirs(tz)
        (dy,) = torch.autograd.grad(y.sum(), tz)
        assert np.abs(ours(z) - y.detach().numpy()).max() < 1e-14
        assert np.abs(ours_d(z) - dy.numpy()).max() < 1e-14


# ------------------------------------------------------------------ whole-loop pins
def _cfg(fw="swiglu", loss="dot", ns=0, renorm=False, order="apply_then_update", chunk=3,
         d=4, dh=8, T=9, lr=(), wd=0.0):
    return Config("t", 1, 1, T, chunk, d, dh, fw, loss, ns, renorm, "f32", order,
                  lr=tuple(lr), weight_decay=wd)


def _rand_problem(cfg, rng, wscale=0.5):
    Ws = _rand_ws(cfg.fw, cfg.dim, cfg.hidden, rng, wscale)
    Q = rng.standard_normal((cfg.seq_len, cfg.dim))
    K, V, eta = _rand_chunk(cfg.seq_len, cfg.dim, rng)
    return Ws, Q, K, V, eta


@pytest.mark.parametrize("fw", ["swiglu", "gelu", "linear"])
@pytest.mark.parametrize("loss", ["dot", "mse"])
@pytest.mark.parametrize("ns,renorm", [(0, False), (0, True), (5, True)])
@pytest.mark.parametrize("order", ["apply_then_update", "update_then_apply"])
def test_matrix_form_matches_per_token_bruteforce(fw, loss, ns, renorm, order):
    cfg = _cfg(fw, loss, ns, renorm, order, chunk=3, d=4, dh=6, T=12)
    Ws, Q, K, V, eta = _rand_problem(cfg, np.random.default_rng(3))
    O1, W1 = orc.sequence_forward(cfg, Ws, Q, K, V, eta)
    O2, W2 = orc.sequence_forward_bruteforce(cfg, Ws, Q, K, V, eta)
    assert np.abs(O1 - O2).max() <= 1e-12 * max(1, np.abs(O2).max())
    for a, b in zip(W1, W2):
        assert np.abs(a - b).max() <= 1e-12 * max(1, np.abs(b).max())


def linear_dot_closed_form_error(order="apply_then_update", chunk=4, T=16, d=5, seed=11):
    """Linear fast weight, inner-product loss, plain SGD, no norm: for any chunking the
    state is W0 + sum_t eta_t v_t k_t^T over the tokens seen, and chunk c's outputs are
    that state applied to its queries (before or after its own tokens, by the order)."""
    cfg = _cfg("linear", "dot", 0, False, order, chunk=chunk, d=d, T=T)
    rng = np.random.default_rng(seed)
    Ws, Q, K, V, eta = _rand_problem(cfg, rng)
    O, Wf = orc.sequence_forward(cfg, Ws, Q, K, V, eta)
    W = Ws[0].copy()
    err = 0.0
    for c in range(T // chunk):
        S = slice(c * chunk, (c + 1) * chunk)
        Wn = W + sum(eta[t] * np.outer(V[t], K[t]) for t in range(c * chunk, (c + 1) * chunk))
        ref = Q[S] @ (W if order == "apply_then_update" else Wn).T
        err = max(err, np.abs(O[S] - ref).max())
        W = Wn
    err = max(err, np.abs(Wf[0] - W).max())
    return err


@pytest.mark.parametrize("order", ["apply_then_update", "update_then_apply"])
@pytest.mark.parametrize("chunk", [1, 4, 16])
def test_linear_dot_closed_form(order, chunk):
    assert linear_dot_closed_form_error(order, chunk) <= 1e-12


def test_scalar_sine_exercise():
    """The TTT-layer explainer's exercise (aivaro.ru page, §10): d = 1, y = w x,
    MSE on predicting the next value from the previous one, SGD with lr 0.01, update on
    the previous token and then output for the current one, over a noisy sine of 1000
    points. As a TTT layer: chunk = 1, k_t = x_{t-1}, v_t = x_t, q_t = x_t, eta_t = 0.01,
    update-then-apply, linear fast weight, MSE loss."""
    rng = np.random.default_rng(5)
    x = np.sin(np.arange(1000) * 0.05) + 0.1 * rng.standard_normal(1000)
    w0 = 0.3
    # the exercise written as a plain scalar loop
    w, outs = w0, []
    for t in range(1, 1000):
        grad = 2.0 * (w * x[t - 1] - x[t]) * x[t - 1]
        w = w - 0.01 * grad
        outs.append(w * x[t])
    cfg = _cfg("linear", "mse", 0, False, "update_then_apply", chunk=1, d=1, T=999)
    O, Wf = orc.sequence_forward(cfg, [np.array([[w0]])], x[1:, None], x[:-1, None],
                                 x[1:, None], np.full(999, 0.01))
    assert np.abs(O[:, 0] - np.array(outs)).max() < 1e-12
    assert abs(Wf[0][0, 0] - w) < 1e-12


@pytest.mark.parametrize("fw,loss", [("swiglu", "dot"), ("gelu", "mse"), ("linear", "dot")])
@pytest.mark.parametrize("ns,renorm", [(0, False), (0, True), (5, True)])
def test_eta_zero_leaves_state_bitwise(fw, loss, ns, renorm):
    cfg = _cfg(fw, loss, ns, renorm, chunk=3, T=9)
    Ws, Q, K, V, eta = _rand_problem(cfg, np.random.default_rng(1))
    O, Wf = orc.sequence_forward(cfg, Ws, Q, K, V, np.zeros_like(eta))
    for a, b in zip(Wf, Ws):
        assert np.array_equal(a, b)
    assert np.array_equal(O, orc.fw_apply(fw, Ws, Q))


def test_shifted_causality():
    """Outputs of chunks <= c do not change when keys, values or eta of chunks >= c
    change (apply-then-update), and chunk 0 is answered by W0."""
    cfg = _cfg("swiglu", "dot", 5, True, chunk=4, T=16, d=4, dh=8)
    rng = np.random.default_rng(2)
    Ws, Q, K, V, eta = _rand_problem(cfg, rng)
    O, _ = orc.sequence_forward(cfg, Ws, Q, K, V, eta)
    assert np.array_equal(O[:4], orc.fw_apply("swiglu", Ws, Q[:4]))
    for c in range(4):
        K2, V2, e2 = K.copy(), V.copy(), eta.copy()
        K2[c * 4:] += 1.0
        V2[c * 4:] -= 1.0
        e2[c * 4:] *= 3.0
        O2, _ = orc.sequence_forward(cfg, Ws, Q, K2, V2, e2)
        assert np.array_equal(O2[:(c + 1) * 4], O[:(c + 1) * 4])
        if c < 3:
            assert not np.array_equal(O2[(c + 1) * 4:], O[(c + 1) * 4:])


def test_block_summation_invariance():
    """Summing a large chunk's gradient block by block gives the one-block result."""
    cfg = _cfg("swiglu", "dot", 5, True, chunk=300, T=600, d=8, dh=16)
    Ws, Q, K, V, eta = _rand_problem(cfg, np.random.default_rng(4), 0.3)
    O1, W1 = orc.sequence_forward(cfg, Ws, Q, K, V, eta, block_rows=None)
    O2, W2 = orc.sequence_forward(cfg, Ws, Q, K, V, eta, block_rows=37)
    assert np.abs(O1 - O2).max() <= 1e-12 * np.abs(O1).max()
    for a, b in zip(W1, W2):
        assert np.abs(a - b).max() <= 1e-12 * np.abs(b).max()


# ------------------------------------------------------------------ Newton-Schulz pins
def ns5_svd_error(shape, seed=0, rank=None):
    """NS5 acts on singular values only: G = U S V^T maps to U phi^5(S/(|G|_F+eps)) V^T
    with phi(s) = a s + b s^3 + c s^5 (each step's X X^T, its square and the product
    with X are diagonal in G's singular bases)."""
    rng = np.random.default_rng(seed)
    G = rng.standard_normal(shape)
    if rank is not None:
        G = rng.standard_normal((shape[0], rank)) @ rng.standard_normal((rank, shape[1]))
    U, S, Vt = np.linalg.svd(G, full_matrices=False)
    s = S / (math.sqrt(float(np.sum(S * S))) + orc.NS_EPS)
    a, b, c = orc.MUON_COEFFS
    for _ in range(5):
        s = a * s + b * s ** 3 + c * s ** 5
    ref = (U * s) @ Vt
    return np.abs(orc.newton_schulz5(G) - ref).max()


@pytest.mark.parametrize("shape", [(6, 9), (9, 6), (7, 7), (32, 64), (64, 32)])
def test_ns5_spectral_closed_form(shape):
    assert ns5_svd_error(shape) < 1e-12


def test_ns5_rank_deficient_and_zero():
    assert ns5_svd_error((12, 20), rank=3) < 1e-12
    assert np.array_equal(orc.newton_schulz5(np.zeros((4, 6))), np.zeros((4, 6)))


def test_ns5_symmetries():
    G = np.random.default_rng(9).standard_normal((16, 24))
    U = orc.newton_schulz5(G)
    assert np.abs(orc.newton_schulz5(-G) + U).max() < 1e-14
    assert np.abs(orc.newton_schulz5(G.T) - U.T).max() < 1e-14
    assert np.abs(orc.newton_schulz5(3.7 * G) - U).max() < 1e-7   # scale-free up to eps


def test_ns5_singular_values_near_one():
    """Muon's iteration pushes every singular value that is not tiny into a band around
    1: for sigma/|G|_F >= 3e-3 the 5-step quintic lands in [0.68, 1.21]."""
    G = np.random.default_rng(10).standard_normal((64, 128))
    S = np.linalg.svd(orc.newton_schulz5(G), compute_uv=False)
    assert S.min() > 0.68 and S.max() < 1.21


# ------------------------------------------------------------------ renorm pins
def test_renorm_restores_row_norms():
    rng = np.random.default_rng(8)
    W = rng.standard_normal((20, 30))
    Wn = W - rng.standard_normal((20, 30))
    R = orc.renorm_rows(W, Wn)
    assert np.abs(np.linalg.norm(R, axis=1) / np.linalg.norm(W, axis=1) - 1).max() < 1e-15
    # direction of every row is that of the updated row
    cos = np.sum(R * Wn, 1) / np.linalg.norm(R, axis=1) / np.linalg.norm(Wn, axis=1)
    assert np.abs(cos - 1).max() < 1e-15


def test_renorm_zero_row_guard():
    W = np.ones((3, 4))
    Wn = W.copy()
    Wn[1] = 0
    R = orc.renorm_rows(W, Wn)
    assert np.array_equal(R[1], np.zeros(4))
    assert np.allclose(R[[0, 2]], W[[0, 2]], rtol=0, atol=1e-15)


def test_sequence_renorm_keeps_initial_norms():
    cfg = _cfg("swiglu", "dot", 5, True, chunk=4, T=20, d=6, dh=10)
    Ws, Q, K, V, eta = _rand_problem(cfg, np.random.default_rng(6))
    _, Wf = orc.sequence_forward(cfg, Ws, Q, K, V, eta)
    for a, b in zip(Wf, Ws):
        assert np.abs(np.linalg.norm(a, axis=1) - np.linalg.norm(b, axis=1)).max() < 1e-13
        assert np.abs(a - b).max() > 1e-3   # the state did move


# ------------------------------------------------------------------ step size, weight decay
def linear_dot_step_closed_form_error(order="apply_then_update", chunk=4, T=16, d=5, seed=12,
                                      lr=0.37, wd=0.15):
    """Linear fast weight, inner-product loss, no Muon, no norm, with step size lr and
    weight decay wd: the chunk gradient is -sum_t eta_t v_t k_t^T in closed form, so the
    state after chunk c is (1 - wd) W_c + lr sum_t eta_t v_t k_t^T, summed token by
    token here."""
    cfg = _cfg("linear", "dot", 0, False, order, chunk=chunk, d=d, T=T, lr=(lr,), wd=wd)
    Ws, Q, K, V, eta = _rand_problem(cfg, np.random.default_rng(seed))
    O, Wf = orc.sequence_forward(cfg, Ws, Q, K, V, eta)
    W = Ws[0].copy()
    err = 0.0
    for c in range(T // chunk):
        S = slice(c * chunk, (c + 1) * chunk)
        step = np.zeros_like(W)
        for t in range(c * chunk, (c + 1) * chunk):
            step += eta[t] * np.outer(V[t], K[t])
        Wn = (1.0 - wd) * W + lr * step
        ref = Q[S] @ (W if order == "apply_then_update" else Wn).T
        err = max(err, np.abs(O[S] - ref).max())
        W = Wn
    return max(err, np.abs(Wf[0] - W).max())


@pytest.mark.parametrize("order", ["apply_then_update", "update_then_apply"])
@pytest.mark.parametrize("lr,wd", [(0.37, 0.15), (2.0, 0.0), (1.0, 0.5)])
def test_linear_dot_step_size_and_decay_closed_form(order, lr, wd):
    assert linear_dot_step_closed_form_error(order, lr=lr, wd=wd) <= 1e-12


@pytest.mark.parametrize("fw,loss", [("swiglu", "dot"), ("gelu", "mse")])
@pytest.mark.parametrize("ns", [0, 5])
def test_decay_alone_is_a_power(fw, loss, ns):
    """eta = 0 makes every gradient (and its orthogonalisation) zero, so with no renorm
    n chunks leave exactly (1 - wd)^n W0."""
    wd = 0.05
    cfg = _cfg(fw, loss, ns, False, chunk=3, T=12, lr=(0.7, 1.3, 0.2), wd=wd)
    Ws, Q, K, V, eta = _rand_problem(cfg, np.random.default_rng(21))
    _, Wf = orc.sequence_forward(cfg, Ws, Q, K, V, np.zeros_like(eta))
    for a, b in zip(Wf, Ws):
        assert np.abs(a - (1.0 - wd) ** 4 * b).max() <= 1e-15 * np.abs(b).max()


def test_decay_alone_is_undone_by_renorm():
    """With the row renorm, a pure decay (eta = 0) is rescaled back to the norms before
    the step: the state does not move."""
    cfg = _cfg("swiglu", "dot", 5, True, chunk=3, T=12, wd=0.3)
    Ws, Q, K, V, eta = _rand_problem(cfg, np.random.default_rng(22))
    _, Wf = orc.sequence_forward(cfg, Ws, Q, K, V, np.zeros_like(eta))
    for a, b in zip(Wf, Ws):
        assert np.abs(a - b).max() <= 1e-14 * np.abs(b).max()


@pytest.mark.parametrize("fw,loss", [("swiglu", "dot"), ("gelu", "mse"), ("swiglu", "mse")])
@pytest.mark.parametrize("renorm", [False, True])
def test_uniform_step_size_equals_scaled_eta_without_muon(fw, loss, renorm):
    """Without Muon the step is lr times a gradient that is linear in eta, so step size c
    with eta is the same run as step size 1 with c eta."""
    c = 0.35
    cfg = _cfg(fw, loss, 0, renorm, chunk=3, T=12, d=4, dh=6, lr=(c, c, c))
    Ws, Q, K, V, eta = _rand_problem(cfg, np.random.default_rng(23))
    O1, W1 = orc.sequence_forward(cfg, Ws, Q, K, V, eta)
    O2, W2 = orc.sequence_forward(cfg.replace(lr=()), Ws, Q, K, V, c * eta)
    assert np.abs(O1 - O2).max() <= 1e-12 * np.abs(O2).max()
    for a, b in zip(W1, W2):
        assert np.abs(a - b).max() <= 1e-12 * np.abs(b).max()


def muon_step_band(lr=(0.3, 0.5, 2.0), seed=24):
    """Muon with step sizes and no norm, one chunk: (W0 - W1) / lr_i is the orthogonalised
    gradient, whose singular values lie in the Newton-Schulz band [0.68, 1.21] whatever
    the gradient's scale (the step size multiplies the orthogonalised step, it is not
    normalised away). Returns the extreme singular values over the matrices."""
    cfg = _cfg("swiglu", "dot", 5, False, chunk=32, T=32, d=8, dh=16, lr=lr)
    Ws, Q, K, V, eta = _rand_problem(cfg, np.random.default_rng(seed))
    _, Wf = orc.sequence_forward(cfg, Ws, Q, K, V, eta)
    lo, hi = np.inf, 0.0
    for a, b, step in zip(Wf, Ws, lr):
        S = np.linalg.svd((b - a) / step, compute_uv=False)
        lo, hi = min(lo, S.min()), max(hi, S.max())
    return lo, hi


def test_muon_step_size_scales_the_orthogonalised_step():
    lo, hi = muon_step_band()
    assert lo > 0.68 and hi < 1.21


# ------------------------------------------------------------------ apply backward
def apply_vjp_fd_error(fw, seed=31, d=4, dh=6, n=5, eps=1e-6):
    """Central finite differences of sum <dO, f_W(Q)> in every entry of Q and of W."""
    rng = np.random.default_rng(seed)
    Ws = _rand_ws(fw, d, dh, rng)
    Q = rng.standard_normal((n, d))
    dO = rng.standard_normal((n, d))
    dQ, dW = orc.apply_vjp(fw, Ws, Q, dO)
    f = lambda Ws_, Q_: float(np.sum(dO * orc.fw_apply(fw, Ws_, Q_)))
    worst = 0.0
    fdq = np.zeros_like(Q)
    for idx in np.ndindex(Q.shape):
        Qp, Qm = Q.copy(), Q.copy()
        Qp[idx] += eps
        Qm[idx] -= eps
        fdq[idx] = (f(Ws, Qp) - f(Ws, Qm)) / (2 * eps)
    worst = max(worst, np.abs(fdq - dQ).max() / np.abs(fdq).max())
    for i, W in enumerate(Ws):
        fd = np.zeros_like(W)
        for idx in np.ndindex(W.shape):
            Wp = [w.copy() for w in Ws]
            Wm = [w.copy() for w in Ws]
            Wp[i][idx] += eps
            Wm[i][idx] -= eps
            fd[idx] = (f(Wp, Q) - f(Wm, Q)) / (2 * eps)
        worst = max(worst, np.abs(fd - dW[i]).max() / np.abs(fd).max())
    return worst


@pytest.mark.parametrize("fw", ["swiglu", "gelu", "linear"])
def test_apply_backward_matches_finite_differences(fw):
    assert apply_vjp_fd_error(fw) < 1e-7


@pytest.mark.parametrize("fw", ["swiglu", "gelu", "linear"])
def test_apply_backward_matches_torch_autograd(fw):
    rng = np.random.default_rng(32)
    Ws = _rand_ws(fw, 6, 10, rng)
    Q = rng.standard_normal((7, 6))
    dO = rng.standard_normal((7, 6))
    dQ, dW = orc.apply_vjp(fw, Ws, Q, dO)
    F = torch.nn.functional
    tq = torch.tensor(Q, requires_grad=True)
    tw = [torch.tensor(w, requires_grad=True) for w in Ws]
    if fw == "swiglu":
        out = (F.silu(tq @ tw[0].T) * (tq @ tw[1].T)) @ tw[2].T
    elif fw == "gelu":
        out = F.gelu(tq @ tw[0].T) @ tw[1].T
    else:
        out = tq @ tw[0].T
    grads = torch.autograd.grad((out * torch.tensor(dO)).sum(), [tq] + tw)
    assert np.abs(grads[0].numpy() - dQ).max() < 1e-12
    for g, w in zip(grads[1:], dW):
        assert np.abs(g.numpy() - w).max() < 1e-12


def test_apply_backward_weights_equal_the_inner_product_gradient_at_eta_minus_one():
    """The weight part of the apply backward is the inner-product loss gradient with keys
    Q, values dO and eta = -1 (the loss is then +sum <f(q), dO>)."""
    rng = np.random.default_rng(33)
    for fw in ("swiglu", "gelu", "linear"):
        Ws = _rand_ws(fw, 5, 9, rng)
        Q = rng.standard_normal((8, 5))
        dO = rng.standard_normal((8, 5))
        _, dW = orc.apply_vjp(fw, Ws, Q, dO)
        g = orc.chunk_gradient(fw, "dot", Ws, Q, dO, -np.ones(8))
        for a, b in zip(dW, g):
            assert np.abs(a - b).max() < 1e-13


# ------------------------------------------------------------------ sampled rows, all problems
SAMPLE_ROWS = np.array([0, 5, 7, 8, 13, 15, 16, 23, 24, 30, 31])


def apply_rows_error(order, seed=41):
    """The apply_rows branch of the sequence loop (it writes stored samples of runs too long
    to keep whole) against the per-token brute force, which computes every row: rows in
    every chunk, each chunk's first and last token among them, token blocks shorter than
    a chunk, and rows outside the sample left at zero."""
    cfg = _cfg("swiglu", "dot", 5, True, order, chunk=8, T=32, d=4, dh=6)
    Ws, Q, K, V, eta = _rand_problem(cfg, np.random.default_rng(seed))
    O, Wf = orc.sequence_forward(cfg, Ws, Q, K, V, eta, block_rows=3, apply_rows=SAMPLE_ROWS)
    Ob, Wb = orc.sequence_forward_bruteforce(cfg, Ws, Q, K, V, eta)
    rest = np.setdiff1d(np.arange(cfg.seq_len), SAMPLE_ROWS)
    if np.any(O[rest] != 0.0):
        return np.inf
    err = np.abs(O[SAMPLE_ROWS] - Ob[SAMPLE_ROWS]).max() / np.abs(Ob).max()
    for a, b in zip(Wf, Wb):
        err = max(err, np.abs(a - b).max() / np.abs(b).max())
    return err


@pytest.mark.parametrize("order", ["apply_then_update", "update_then_apply"])
def test_apply_rows_match_the_bruteforce_rows(order):
    assert apply_rows_error(order) <= 1e-12


def forward_all_error(seed=1234):
    """forward_all over a batch of 2 and 3 heads against the per-token brute force run on
    each problem's own inputs regenerated alone (its token blocks, and its head's initial
    weights), so that a wrong head, batch element or tensor fails."""
    import ttt_inputs as ti
    cfg = Config("fa", 2, 3, 12, 4, 4, 6, "swiglu", "dot", 5, True, "f32",
                 "apply_then_update", seed)
    res = orc.forward_all(cfg, ti.make_inputs(cfg))
    weights = ti.make_weights(cfg)
    err = 0.0
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            p = ti.make_problem_inputs(cfg, b, h)
            Ob, Wb = orc.sequence_forward_bruteforce(cfg, [w[h] for w in weights], p["q"], p["k"],
                                                     p["v"], p["eta"])
            Og, Wg = res[(b, h)]
            err = max(err, np.abs(Og - Ob).max() / np.abs(Ob).max())
            for a, c in zip(Wg, Wb):
                err = max(err, np.abs(a - c).max() / np.abs(c).max())
    return err


def test_forward_all_runs_each_problem_on_its_own_inputs():
    assert forward_all_error() <= 1e-12


# ------------------------------------------------------------------ chunks that do not update
MASKS = [(0, 1, 0, 1), (1, 0, 0, 1), (0, 0, 0, 0), (1, 1, 1, 1), (1, 0, 1, 0)]


def masked_linear_closed_form_error(order, mask, chunk=3, T=12, d=4, seed=13, lr=0.6, wd=0.1):
    """Linear fast weight, inner-product loss, no Muon, no norm: only the chunks whose flag
    is set move the state, each to (1 - wd) W + lr sum_t eta_t v_t k_t^T over its own
    tokens (summed token by token here); a chunk without the flag is answered by the state
    as it stands and neither steps nor decays it."""
    cfg = _cfg("linear", "dot", 0, False, order, chunk=chunk, d=d, T=T, lr=(lr,), wd=wd)
    Ws, Q, K, V, eta = _rand_problem(cfg, np.random.default_rng(seed))
    O, Wf = orc.sequence_forward(cfg, Ws, Q, K, V, eta, update_chunks=mask)
    W = Ws[0].copy()
    err = 0.0
    for c in range(T // chunk):
        S = slice(c * chunk, (c + 1) * chunk)
        Wn = W
        if mask[c]:
            step = np.zeros_like(W)
            for t in range(c * chunk, (c + 1) * chunk):
                step += eta[t] * np.outer(V[t], K[t])
            Wn = (1.0 - wd) * W + lr * step
        ref = Q[S] @ (W if order == "apply_then_update" else Wn).T
        err = max(err, np.abs(O[S] - ref).max())
        W = Wn
    return max(err, np.abs(Wf[0] - W).max())


@pytest.mark.parametrize("order", ["apply_then_update", "update_then_apply"])
@pytest.mark.parametrize("mask", MASKS)
def test_update_flags_linear_closed_form(order, mask):
    assert masked_linear_closed_form_error(order, mask) <= 1e-12


@pytest.mark.parametrize("fw,loss", [("swiglu", "dot"), ("gelu", "mse"), ("linear", "mse")])
@pytest.mark.parametrize("order", ["apply_then_update", "update_then_apply"])
def test_update_flags_match_the_bruteforce(fw, loss, order):
    cfg = _cfg(fw, loss, 5 if fw != "linear" else 0, True, order, chunk=3, d=4, dh=6, T=12)
    Ws, Q, K, V, eta = _rand_problem(cfg, np.random.default_rng(14))
    for mask in MASKS:
        O1, W1 = orc.sequence_forward(cfg, Ws, Q, K, V, eta, update_chunks=mask)
        O2, W2 = orc.sequence_forward_bruteforce(cfg, Ws, Q, K, V, eta, update_chunks=mask)
        assert np.abs(O1 - O2).max() <= 1e-12 * max(1, np.abs(O2).max())
        for a, b in zip(W1, W2):
            assert np.abs(a - b).max() <= 1e-12 * max(1, np.abs(b).max())


@pytest.mark.parametrize("ns,renorm", [(0, False), (5, True)])
def test_a_chunk_without_update_equals_eta_zero(ns, renorm):
    """With no weight decay, a chunk that does not update is the same run as that chunk's
    eta set to zero (a zero gradient, and NS5(0) = 0, leave the state bitwise), and all
    flags set is the run with no flags."""
    cfg = _cfg("swiglu", "dot", ns, renorm, chunk=3, T=12, d=4, dh=6)
    Ws, Q, K, V, eta = _rand_problem(cfg, np.random.default_rng(15))
    mask = (1, 0, 1, 0)
    O1, W1 = orc.sequence_forward(cfg, Ws, Q, K, V, eta, update_chunks=mask)
    e0 = eta.copy()
    for c, m in enumerate(mask):
        if not m:
            e0[c * 3:(c + 1) * 3] = 0.0
    O2, W2 = orc.sequence_forward(cfg, Ws, Q, K, V, e0)
    assert np.array_equal(O1, O2)
    for a, b in zip(W1, W2):
        assert np.array_equal(a, b)
    O3, W3 = orc.sequence_forward(cfg, Ws, Q, K, V, eta, update_chunks=(1, 1, 1, 1))
    O4, W4 = orc.sequence_forward(cfg, Ws, Q, K, V, eta)
    assert np.array_equal(O3, O4) and all(np.array_equal(a, b) for a, b in zip(W3, W4))


# ------------------------------------------------------------------ momentum over chunks
def momentum_linear_closed_form_error(order="apply_then_update", beta=0.6, lr=0.7, wd=0.1,
                                      chunk=3, T=12, d=4, seed=16):
    """Linear fast weight, inner-product loss, no Muon, no norm, heavy-ball momentum: the
    buffer is M_c = beta M_{c-1} + g_c with g_c = -sum_t eta_t v_t k_t^T over chunk c's
    tokens (summed token by token here), and W_c = (1 - wd) W_{c-1} - lr M_c; the returned
    state is W followed by M."""
    cfg = _cfg("linear", "dot", 0, False, order, chunk=chunk, d=d, T=T, lr=(lr,), wd=wd)
    cfg = cfg.replace(momentum=beta)
    Ws, Q, K, V, eta = _rand_problem(cfg, np.random.default_rng(seed))
    O, out = orc.sequence_forward(cfg, Ws, Q, K, V, eta)
    W, M = Ws[0].copy(), np.zeros_like(Ws[0])
    err = 0.0
    for c in range(T // chunk):
        S = slice(c * chunk, (c + 1) * chunk)
        g = np.zeros_like(W)
        for t in range(c * chunk, (c + 1) * chunk):
            g -= eta[t] * np.outer(V[t], K[t])
        M = beta * M + g
        Wn = (1.0 - wd) * W - lr * M
        ref = Q[S] @ (W if order == "apply_then_update" else Wn).T
        err = max(err, np.abs(O[S] - ref).max())
        W = Wn
    err = max(err, np.abs(out[0] - W).max())
    if not beta:                       # no momentum: the state is the fast weights alone
        return err if len(out) == 1 else np.inf
    return max(err, np.abs(out[1] - M).max())


@pytest.mark.parametrize("order", ["apply_then_update", "update_then_apply"])
@pytest.mark.parametrize("beta", [0.0, 0.5, 0.9])
def test_momentum_linear_closed_form(order, beta):
    assert momentum_linear_closed_form_error(order, beta) <= 1e-12


@pytest.mark.parametrize("fw,loss,ns,renorm", [("swiglu", "dot", 5, True),
                                               ("gelu", "mse", 0, False),
                                               ("swiglu", "mse", 5, False)])
def test_momentum_matches_the_bruteforce(fw, loss, ns, renorm):
    cfg = _cfg(fw, loss, ns, renorm, chunk=3, d=4, dh=6, T=12).replace(momentum=0.7)
    Ws, Q, K, V, eta = _rand_problem(cfg, np.random.default_rng(17))
    O1, W1 = orc.sequence_forward(cfg, Ws, Q, K, V, eta)
    O2, W2 = orc.sequence_forward_bruteforce(cfg, Ws, Q, K, V, eta)
    assert len(W1) == 2 * len(Ws) == len(W2)
    assert np.abs(O1 - O2).max() <= 1e-12 * max(1, np.abs(O2).max())
    for a, b in zip(W1, W2):
        assert np.abs(a - b).max() <= 1e-12 * max(1, np.abs(b).max())


def muon_momentum_band(beta=0.8, lr=(0.3, 0.5, 2.0), seed=25):
    """Muon on the momentum buffer, no norm: each chunk's step (W_prev - W) / lr_i is
    NS5 of the buffer, whose singular values lie in the Newton-Schulz band. Returns the
    extreme singular values over chunks and matrices."""
    cfg = _cfg("swiglu", "dot", 5, False, chunk=8, T=24, d=6, dh=12, lr=lr).replace(
        momentum=beta)
    Ws, Q, K, V, eta = _rand_problem(cfg, np.random.default_rng(seed))
    lo, hi = np.inf, 0.0
    prev = Ws
    for c in range(3):
        _, out = orc.sequence_forward(cfg, Ws, Q, K, V, eta, n_chunks=c + 1)
        cur = out[:3]
        for a, b, step in zip(cur, prev, lr):
            S = np.linalg.svd((b - a) / step, compute_uv=False)
            lo, hi = min(lo, S.min()), max(hi, S.max())
        prev = cur
    return lo, hi


def test_muon_orthogonalises_the_momentum_buffer():
    lo, hi = muon_momentum_band()
    assert lo > 0.68 and hi < 1.21


# ------------------------------------------------------------------ mutation tests
def _all_pins_pass():
    try:
        return _all_pins_pass_inner()
    except (ValueError, IndexError):   # a shape error is a caught mistake too
        return False


def _all_pins_pass_inner():
    checks = [
        fd_gradient_error("swiglu", "dot") < 1e-6,
        fd_gradient_error("swiglu", "mse") < 1e-6,
        fd_gradient_error("gelu", "mse") < 1e-6,
        linear_dot_closed_form_error("apply_then_update") <= 1e-12,
        linear_dot_closed_form_error("update_then_apply") <= 1e-12,
        ns5_svd_error((6, 9)) < 1e-12,
        ns5_svd_error((9, 6)) < 1e-12,
    ]
    W = np.random.default_rng(1).standard_normal((5, 7))
    Wn = W + np.random.default_rng(2).standard_normal((5, 7))
    R = orc.renorm_rows(W, Wn)
    checks.append(np.abs(np.linalg.norm(R, axis=1) - np.linalg.norm(W, axis=1)).max() < 1e-14)
    checks.append(linear_dot_step_closed_form_error("apply_then_update") <= 1e-12)
    lo, hi = muon_step_band()
    checks.append(lo > 0.68 and hi < 1.21)
    checks.append(apply_rows_error("apply_then_update") <= 1e-12)
    checks.append(apply_rows_error("update_then_apply") <= 1e-12)
    checks.append(forward_all_error() <= 1e-12)
    for order in ("apply_then_update", "update_then_apply"):
        checks.append(masked_linear_closed_form_error(order, (0, 1, 0, 1)) <= 1e-12)
        checks.append(masked_linear_closed_form_error(order, (1, 0, 0, 1)) <= 1e-12)
        checks.append(momentum_linear_closed_form_error(order) <= 1e-12)
    lo, hi = muon_momentum_band()
    checks.append(lo > 0.68 and hi < 1.21)
    return all(checks)


def test_pins_pass_on_the_unmutated_oracle():
    assert _all_pins_pass()


def _mut_silu_prime(z):  # dropped term of silu'
    return orc.sigmoid(z)


def _mut_output_error(loss, F_k, V, eta):  # sign error in the inner-product error
    return eta[:, None] * V if loss == "dot" else 2.0 * eta[:, None] * (F_k - V)


def _mut_ns(G, steps=5, coeffs=orc.MUON_COEFFS, eps=orc.NS_EPS):  # A instead of A^2
    a, b, c = coeffs
    X = G / (np.linalg.norm(G) + eps)
    wide = X.shape[0] <= X.shape[1]
    X = X if wide else X.T
    for _ in range(steps):
        A = X @ X.T
        X = a * X + (b * A + c * A) @ X
    return X if wide else X.T


def _mut_ns_transpose(G, steps=5, coeffs=orc.MUON_COEFFS, eps=orc.NS_EPS):  # no undo
    a, b, c = coeffs
    X = G / (np.linalg.norm(G) + eps)
    if X.shape[0] > X.shape[1]:
        X = X.T
    for _ in range(steps):
        A = X @ X.T
        X = a * X + (b * A + c * A @ A) @ X
    return X


def _mut_renorm(W_prev, W_new):  # renormalises to unit norm
    return W_new / np.linalg.norm(W_new, axis=1, keepdims=True)


def _mut_block_grad_transposed(fw, loss, Ws, K, V, eta):  # g2 = H^T E instead of E^T H
    g = _ORIG_BLOCK(fw, loss, Ws, K, V, eta)
    if fw == "swiglu":
        g[2] = g[2][::-1]
    return g


_ORIG_BLOCK = orc._block_gradient


def _mut_decay_after_step(Ws, grads, ns_steps, renorm, lr=None, weight_decay=0.0):
    # the decay applied to the stepped state instead of before the step
    steps = [1.0] * len(Ws) if lr is None else list(lr)
    out = []
    for W, g, step in zip(Ws, grads, steps):
        U = orc.newton_schulz5(g, ns_steps) if ns_steps > 0 else g
        W_new = (1.0 - weight_decay) * (W - step * U)
        out.append(orc.renorm_rows(W, W_new) if renorm else W_new)
    return out


def _mut_step_before_ns(Ws, grads, ns_steps, renorm, lr=None, weight_decay=0.0):
    # the step size applied to the gradient before the orthogonalisation
    steps = [1.0] * len(Ws) if lr is None else list(lr)
    out = []
    for W, g, step in zip(Ws, grads, steps):
        U = orc.newton_schulz5(step * g, ns_steps) if ns_steps > 0 else step * g
        W_new = (1.0 - weight_decay) * W - U
        out.append(orc.renorm_rows(W, W_new) if renorm else W_new)
    return out


_ORIG_SEQ = orc.sequence_forward


def _mut_rows_offset(cfg, W0s, Q, K, V, eta, block_rows=8192, apply_rows=None, n_chunks=None,
                     update_chunks=None):
    # the sampled rows of chunk c answered with the queries at (row - chunk start)
    if apply_rows is not None:
        Q = np.array(Q, np.float64)
        rows = np.asarray(apply_rows)
        Q[rows] = Q[rows - (rows // cfg.chunk) * cfg.chunk]
    return _ORIG_SEQ(cfg, W0s, Q, K, V, eta, block_rows, apply_rows, n_chunks, update_chunks)


def _mut_mask_ignored(cfg, W0s, Q, K, V, eta, block_rows=8192, apply_rows=None, n_chunks=None,
                      update_chunks=None):
    # every chunk updates whatever its flag says
    return _ORIG_SEQ(cfg, W0s, Q, K, V, eta, block_rows, apply_rows, n_chunks, None)


def _mut_mask_shifted(cfg, W0s, Q, K, V, eta, block_rows=8192, apply_rows=None, n_chunks=None,
                      update_chunks=None):
    # chunk c takes chunk c-1's flag
    if update_chunks is not None:
        update_chunks = [True] + list(update_chunks)[:-1]
    return _ORIG_SEQ(cfg, W0s, Q, K, V, eta, block_rows, apply_rows, n_chunks, update_chunks)


def _mut_forward_all_head(cfg, inputs, problems=None, block_rows=8192):
    # the initial weights indexed by the batch element instead of the head
    out = {}
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            W0s = [w[b % cfg.heads] for w in inputs["w0"]]
            out[(b, h)] = orc.sequence_forward(cfg, W0s, inputs["q"][b, h], inputs["k"][b, h],
                                               inputs["v"][b, h], inputs["eta"][b, h], block_rows)
    return out


def _mut_forward_all_qk(cfg, inputs, problems=None, block_rows=8192):
    # keys passed where the queries go
    out = {}
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            W0s = [w[h] for w in inputs["w0"]]
            out[(b, h)] = orc.sequence_forward(cfg, W0s, inputs["k"][b, h], inputs["k"][b, h],
                                               inputs["v"][b, h], inputs["eta"][b, h], block_rows)
    return out


def _mut_momentum_on_g(Ms, grads, beta):      # beta scales the new gradient, not the buffer
    return [np.asarray(M, np.float64) + beta * g for M, g in zip(Ms, grads)]


@pytest.mark.parametrize("name,target,mut", [
    ("silu' term", "silu_prime", _mut_silu_prime),
    ("error sign", "_output_error", _mut_output_error),
    ("NS square", "newton_schulz5", _mut_ns),
    ("NS transpose", "newton_schulz5", _mut_ns_transpose),
    ("renorm target", "renorm_rows", _mut_renorm),
    ("g2 index", "_block_gradient", _mut_block_grad_transposed),
    ("decay after the step", "update_state", _mut_decay_after_step),
    ("step size before NS", "update_state", _mut_step_before_ns),
    ("sampled rows offset", "sequence_forward", _mut_rows_offset),
    ("forward_all head index", "forward_all", _mut_forward_all_head),
    ("forward_all keys as queries", "forward_all", _mut_forward_all_qk),
    ("update flags ignored", "sequence_forward", _mut_mask_ignored),
    ("update flags shifted", "sequence_forward", _mut_mask_shifted),
    ("momentum on the gradient", "momentum_step", _mut_momentum_on_g),
])
def test_planted_mistake_is_caught(monkeypatch, name, target, mut):
    monkeypatch.setattr(orc, target, mut)
    assert not _all_pins_pass(), name
