"""Pins of the oracle's backward through one chunk's update (chunk_vjp and its parts).

Two independent routes to the same numbers: central finite differences of the chunk map,
and torch autograd in fp64 on a torch transcription of the forward whose inner gradient is
itself taken by autograd (create_graph), so that no hand-derived second derivative is
shared with the oracle. Planted mistakes at the end check that each plausible slip fails.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle.ttt_oracle as orc
from ttt_inputs import Config


def _cfg(fw, loss, ns, renorm, order="apply_then_update", chunk=3, d=3, dh=4, lr=(), wd=0.0,
         mom=0.0):
    return Config("b", 1, 1, chunk, chunk, d, dh, fw, loss, ns, renorm, "f32", order,
                  lr=tuple(lr), weight_decay=wd, momentum=mom)


def _problem(cfg, seed, wscale=0.6):
    rng = np.random.default_rng(seed)
    shapes = cfg.matrix_shapes() if cfg.fw != "linear" else [(cfg.dim, cfg.dim)]
    if cfg.momentum:       # the state: the matrices, then their momentum buffers
        shapes = shapes + shapes
    Ws = [rng.standard_normal(s) * wscale for s in shapes]
    n, d = cfg.chunk, cfg.dim
    Q, K, V = (rng.standard_normal((n, d)) for _ in range(3))
    eta = 0.05 + 0.3 * rng.random(n)
    dO = rng.standard_normal((n, d))
    dWn = [rng.standard_normal(s) for s in shapes]
    return Ws, Q, K, V, eta, dO, dWn


def _objective(cfg, Ws, Q, K, V, eta, dO, dWn, update=True):
    O, Wn = orc.chunk_step(cfg, Ws, Q, K, V, eta, update)
    return float(np.sum(dO * O) + sum(np.sum(a * b) for a, b in zip(dWn, Wn)))


def chunk_vjp_fd_error(cfg, seed=0, eps=1e-6, update=True):
    Ws, Q, K, V, eta, dO, dWn = _problem(cfg, seed)
    dQ, dK, dV, deta, dW = orc.chunk_vjp(cfg, Ws, Q, K, V, eta, dO, dWn, update)
    args = {"Q": Q, "K": K, "V": V, "eta": eta}
    got = {"Q": dQ, "K": dK, "V": dV, "eta": deta}
    worst = 0.0

    def f(**kw):
        a = dict(args, **{k: v for k, v in kw.items() if k in args})
        return _objective(cfg, kw.get("Ws", Ws), a["Q"], a["K"], a["V"], a["eta"], dO, dWn,
                          update)

    for name, x in args.items():
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            fd[idx] = (f(**{name: xp}) - f(**{name: xm})) / (2 * eps)
        scale = max(np.abs(fd).max(), 1e-3)
        worst = max(worst, np.abs(fd - got[name]).max() / scale)
    for i, W in enumerate(Ws):
        fd = np.zeros_like(W)
        for idx in np.ndindex(W.shape):
            Wp = [w.copy() for w in Ws]
            Wm = [w.copy() for w in Ws]
            Wp[i][idx] += eps
            Wm[i][idx] -= eps
            fd[idx] = (f(Ws=Wp) - f(Ws=Wm)) / (2 * eps)
        worst = max(worst, np.abs(fd - dW[i]).max() / max(np.abs(fd).max(), 1e-3))
    return worst


CASES = list(itertools.product(["swiglu", "gelu", "linear"], ["dot", "mse"],
                               [(0, False), (0, True), (5, True), (5, False)],
                               ["apply_then_update", "update_then_apply"]))


@pytest.mark.parametrize("fw,loss,nsr,order", CASES)
def test_chunk_vjp_matches_finite_differences(fw, loss, nsr, order):
    cfg = _cfg(fw, loss, nsr[0], nsr[1], order)
    assert chunk_vjp_fd_error(cfg) < 1e-6


def test_chunk_vjp_step_size_decay_and_skipped_chunk():
    cfg = _cfg("swiglu", "dot", 5, True, lr=(0.4, 1.3, 0.7), wd=0.1)
    assert chunk_vjp_fd_error(cfg, seed=1) < 1e-6
    assert chunk_vjp_fd_error(_cfg("gelu", "mse", 5, True), seed=2, update=False) < 1e-6


# ------------------------------------------------------------------ torch autograd, fp64
def _torch_chunk(cfg, Ws, Q, K, V, eta):
    Fn = torch.nn.functional

    def f(Wt, X):
        if cfg.fw == "swiglu":
            return (Fn.silu(X @ Wt[0].T) * (X @ Wt[1].T)) @ Wt[2].T
        if cfg.fw == "gelu":
            return Fn.gelu(X @ Wt[0].T) @ Wt[1].T
        return X @ Wt[0].T

    Fk = f(Ws, K)
    if cfg.loss == "dot":
        L = -(eta * (Fk * V).sum(1)).sum()
    else:
        L = (eta * ((Fk - V) ** 2).sum(1)).sum()
    grads = torch.autograd.grad(L, Ws, create_graph=True)
    a, b, c = orc.MUON_COEFFS
    new = []
    for W, g, step in zip(Ws, grads, cfg.step_sizes()):
        U = g
        if cfg.ns_steps:
            X = g / (torch.linalg.norm(g) + orc.NS_EPS)
            tall = X.shape[0] > X.shape[1]
            if tall:
                X = X.T
            for _ in range(cfg.ns_steps):
                A = X @ X.T
                X = a * X + (b * A + c * A @ A) @ X
            U = X.T if tall else X
        Y = (1 - cfg.weight_decay) * W - step * U
        if cfg.renorm:
            Y = Y * (torch.linalg.norm(W, dim=1) / torch.linalg.norm(Y, dim=1))[:, None]
        new.append(Y)
    O = f(Ws if cfg.order == "apply_then_update" else new, Q)
    return O, new


@pytest.mark.parametrize("fw,loss,nsr,order", CASES)
def test_chunk_vjp_matches_torch_autograd(fw, loss, nsr, order):
    cfg = _cfg(fw, loss, nsr[0], nsr[1], order, chunk=5, d=4, dh=6, lr=(0.8, 1.1, 0.9), wd=0.05)
    Ws, Q, K, V, eta, dO, dWn = _problem(cfg, 7)
    dQ, dK, dV, deta, dW = orc.chunk_vjp(cfg, Ws, Q, K, V, eta, dO, dWn)
    t = lambda x: torch.tensor(x, dtype=torch.float64, requires_grad=True)
    tW = [t(w) for w in Ws]
    tq, tk, tv, te = t(Q), t(K), t(V), t(eta)
    O, new = _torch_chunk(cfg, tW, tq, tk, tv, te)
    obj = (O * torch.tensor(dO)).sum() + sum((n * torch.tensor(d)).sum() for n, d in zip(new, dWn))
    g = torch.autograd.grad(obj, [tq, tk, tv, te] + tW)
    ours = [dQ, dK, dV, deta] + dW
    for a, b in zip(ours, g):
        ref = b.numpy()
        assert np.abs(a - ref).max() <= 1e-10 * max(1.0, np.abs(ref).max())


# ------------------------------------------------------------------ parts and the sequence
def test_newton_schulz_vjp_matches_autograd():
    rng = np.random.default_rng(9)
    for shape in [(4, 7), (7, 4), (5, 5)]:
        G = rng.standard_normal(shape)
        dU = rng.standard_normal(shape)
        tg = torch.tensor(G, requires_grad=True)
        a, b, c = orc.MUON_COEFFS
        X = tg / (torch.linalg.norm(tg) + orc.NS_EPS)
        tall = shape[0] > shape[1]
        X = X.T if tall else X
        for _ in range(5):
            A = X @ X.T
            X = a * X + (b * A + c * A @ A) @ X
        U = X.T if tall else X
        (ref,) = torch.autograd.grad((U * torch.tensor(dU)).sum(), tg)
        ours = orc.newton_schulz5_vjp(G, dU)
        assert np.abs(ours - ref.numpy()).max() <= 1e-10 * np.abs(ref.numpy()).max()


def test_renorm_vjp_zero_row_passes_through():
    W = np.array([[1.0, 2.0], [3.0, -1.0]])
    Y = np.array([[0.0, 0.0], [1.0, 1.0]])
    d = np.array([[0.5, -0.25], [1.0, 2.0]])
    dW, dY = orc.renorm_rows_vjp(W, Y, d)
    assert np.array_equal(dY[0], d[0]) and np.array_equal(dW[0], [0.0, 0.0])


def sequence_vjp_fd_error(update_chunks=None, seed=3, eps=1e-6, mom=0.0,
                          order="apply_then_update"):
    cfg = Config("s", 1, 1, 9, 3, 3, 4, "swiglu", "dot", 5, True, "f32", order, momentum=mom)
    rng = np.random.default_rng(seed)
    Ws = [rng.standard_normal(s) * 0.6 for s in cfg.matrix_shapes()]
    Q, K, V = (rng.standard_normal((9, 3)) for _ in range(3))
    eta = 0.05 + 0.3 * rng.random(9)
    dO = rng.standard_normal((9, 3))
    # the cotangent of the final state (with momentum: of the buffers too)
    dWf = [rng.standard_normal(s) for s in cfg.matrix_shapes() * (2 if mom else 1)]

    def obj(Ws_, K_):
        O, Wf = orc.sequence_forward(cfg, Ws_, Q, K_, V, eta, update_chunks=update_chunks)
        return float(np.sum(dO * O) + sum(np.sum(a * b) for a, b in zip(dWf, Wf)))

    _, dK, _, _, dW = orc.sequence_vjp(cfg, Ws, Q, K, V, eta, dO, dWf, update_chunks)
    fdk = np.zeros_like(K)
    for idx in np.ndindex(K.shape):
        Kp, Km = K.copy(), K.copy()
        Kp[idx] += eps
        Km[idx] -= eps
        fdk[idx] = (obj(Ws, Kp) - obj(Ws, Km)) / (2 * eps)
    err = np.abs(fdk - dK).max() / np.abs(fdk).max()
    fdw = np.zeros_like(Ws[2])
    for idx in np.ndindex(Ws[2].shape):
        Wp = [w.copy() for w in Ws]
        Wm = [w.copy() for w in Ws]
        Wp[2][idx] += eps
        Wm[2][idx] -= eps
        fdw[idx] = (obj(Wp, K) - obj(Wm, K)) / (2 * eps)
    return max(err, np.abs(fdw - dW[2]).max() / np.abs(fdw).max())


@pytest.mark.parametrize("mask", [None, (1, 0, 1), (0, 1, 1)])
def test_sequence_vjp_matches_finite_differences(mask):
    assert sequence_vjp_fd_error(mask) < 1e-6


@pytest.mark.parametrize("order", ["apply_then_update", "update_then_apply"])
@pytest.mark.parametrize("nsr", [(5, True), (0, False)])
def test_chunk_vjp_with_momentum_matches_finite_differences(order, nsr):
    # every entry of the state, the momentum buffers included, perturbed
    cfg = _cfg("swiglu", "dot", nsr[0], nsr[1], order, lr=(0.7, 1.3, 0.9), wd=0.03, mom=0.6)
    assert chunk_vjp_fd_error(cfg, seed=4) < 1e-6


@pytest.mark.parametrize("order", ["apply_then_update", "update_then_apply"])
def test_sequence_vjp_with_momentum_matches_finite_differences(order):
    # finite differences of sequence_forward itself (its momentum pinned by its own tests)
    assert sequence_vjp_fd_error((1, 0, 1), seed=5, mom=0.6, order=order) < 1e-6
    assert sequence_vjp_fd_error(None, seed=6, mom=0.3, order=order) < 1e-6


def test_chunk_step_with_momentum_chains_to_the_sequence_forward():
    cfg = Config("s", 1, 1, 12, 4, 3, 4, "swiglu", "dot", 5, True, "f32", "update_then_apply",
                 momentum=0.5)
    rng = np.random.default_rng(8)
    W0 = [rng.standard_normal(s) * 0.6 for s in cfg.matrix_shapes()]
    Q, K, V = (rng.standard_normal((12, 3)) for _ in range(3))
    eta = 0.05 + 0.3 * rng.random(12)
    O, Wf = orc.sequence_forward(cfg, W0, Q, K, V, eta)
    state = W0 + [np.zeros_like(w) for w in W0]
    for c in range(3):
        S = slice(4 * c, 4 * c + 4)
        Oc, state = orc.chunk_step(cfg, state, Q[S], K[S], V[S], eta[S])
        assert np.array_equal(Oc, O[S])
    assert len(state) == 6 and all(np.array_equal(a, b) for a, b in zip(state, Wf))


# ------------------------------------------------------------------ planted mistakes
def _pins_pass():
    checks = [
        chunk_vjp_fd_error(_cfg("swiglu", "dot", 5, True)) < 1e-6,
        chunk_vjp_fd_error(_cfg("swiglu", "mse", 0, True, "update_then_apply")) < 1e-6,
        chunk_vjp_fd_error(_cfg("gelu", "dot", 0, False)) < 1e-6,
        chunk_vjp_fd_error(_cfg("gelu", "mse", 5, False, "update_then_apply")) < 1e-6,
        sequence_vjp_fd_error((1, 0, 1)) < 1e-6,
        chunk_vjp_fd_error(_cfg("swiglu", "dot", 5, True, mom=0.6), seed=4) < 1e-6,
    ]
    return all(checks)


def test_pins_pass_on_the_unmutated_oracle():
    assert _pins_pass()


_ORIG_NS_VJP = orc.newton_schulz5_vjp
_ORIG_RENORM_VJP = orc.renorm_rows_vjp
_ORIG_GRAD_VJP = orc.gradient_vjp
_ORIG_CHUNK_VJP = orc.chunk_vjp


def _mut_silu_second(z):          # a dropped term of silu''
    s = orc.sigmoid(z)
    return s * (1.0 - s) * 2.0


def _mut_gelu_second(z):          # phi(z) alone
    return np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)


def _mut_ns_vjp(G, dU, steps=5, coeffs=orc.MUON_COEFFS, eps=orc.NS_EPS):
    # the Gram's cotangent taken as dA X instead of (dA + dA^T) X
    a, b, c = coeffs
    nrm = np.linalg.norm(G)
    X = G / (nrm + eps)
    dX = np.asarray(dU, np.float64)
    wide = X.shape[0] <= X.shape[1]
    if not wide:
        X, dX = X.T, dX.T
    its = []
    for _ in range(steps):
        its.append(X)
        A = X @ X.T
        X = a * X + (b * A + c * (A @ A)) @ X
    for X in reversed(its):
        A = X @ X.T
        B = b * A + c * (A @ A)
        dB = dX @ X.T
        dA = b * dB + c * (dB @ A + A @ dB)
        dX = a * dX + B.T @ dX + dA @ X
    if not wide:
        dX = dX.T
    return dX / (nrm + eps) - G * (np.sum(G * dX) / (nrm * (nrm + eps) ** 2))


def _mut_renorm_vjp(W_prev, W_new, dOut):    # the reference norm's term dropped
    dW, dY = _ORIG_RENORM_VJP(W_prev, W_new, dOut)
    return np.zeros_like(dW), dY


def _mut_grad_vjp_mse(fw, loss, Ws, K, V, eta, dG):
    # the MSE error held fixed: the terms through its dependence on f(k) dropped
    dW, dK, dV, deta = _ORIG_GRAD_VJP(fw, loss, Ws, K, V, eta, dG)
    if loss != "mse":
        return dW, dK, dV, deta
    dKf, dWf = orc.apply_vjp(fw, Ws, K, -dV)   # dV = -C, C the cotangent reaching f(k)
    return [a - b for a, b in zip(dW, dWf)], dK - dKf, dV, deta


def _mut_chunk_vjp_old_state(cfg, Ws, Q, K, V, eta, dO, dWs_new, update=True):
    # update-then-apply answered as if with the state before the update
    if cfg.order == orc.UPDATE_THEN_APPLY and update:
        c2 = cfg.replace(order=orc.APPLY_THEN_UPDATE)
        return _ORIG_CHUNK_VJP(c2, Ws, Q, K, V, eta, dO, dWs_new, update)
    return _ORIG_CHUNK_VJP(cfg, Ws, Q, K, V, eta, dO, dWs_new, update)


def _mut_chunk_vjp_momentum_beta(cfg, Ws, Q, K, V, eta, dO, dWs_new, update=True):
    # the buffer before the chunk given the cotangent of the new buffer without beta
    out = _ORIG_CHUNK_VJP(cfg, Ws, Q, K, V, eta, dO, dWs_new, update)
    if not cfg.momentum:
        return out
    nm = len(Ws) // 2
    return out[:4] + (out[4][:nm] + [x / cfg.momentum for x in out[4][nm:]],)


def _mut_chunk_vjp_momentum_bypass(cfg, Ws, Q, K, V, eta, dO, dWs_new, update=True):
    # the new buffer's given cotangent passed to the old buffer only, not to the gradient
    if not cfg.momentum:
        return _ORIG_CHUNK_VJP(cfg, Ws, Q, K, V, eta, dO, dWs_new, update)
    nm = len(Ws) // 2
    zero = list(dWs_new[:nm]) + [np.zeros_like(x) for x in dWs_new[nm:]]
    out = _ORIG_CHUNK_VJP(cfg, Ws, Q, K, V, eta, dO, zero, update)
    return out[:4] + (out[4][:nm] + [a + cfg.momentum * np.asarray(b)
                                     for a, b in zip(out[4][nm:], dWs_new[nm:])],)


@pytest.mark.parametrize("name,target,mut", [
    ("momentum beta", "chunk_vjp", _mut_chunk_vjp_momentum_beta),
    ("momentum bypass", "chunk_vjp", _mut_chunk_vjp_momentum_bypass),
    ("silu'' term", "silu_second", _mut_silu_second),
    ("gelu'' term", "gelu_second", _mut_gelu_second),
    ("Gram transpose", "newton_schulz5_vjp", _mut_ns_vjp),
    ("renorm reference", "renorm_rows_vjp", _mut_renorm_vjp),
    ("MSE error held fixed", "gradient_vjp", _mut_grad_vjp_mse),
    ("state of the apply", "chunk_vjp", _mut_chunk_vjp_old_state),
])
def test_planted_mistake_is_caught(monkeypatch, name, target, mut):
    monkeypatch.setattr(orc, target, mut)
    assert not _pins_pass(), name
