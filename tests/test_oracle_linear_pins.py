"""Pins of the TTT-Linear oracle against facts that do not come from the oracle itself.

The variant is the ablated TTT-Linear of "One-Minute Video Generation with
Test-Time Training" (paper-notes page, ablation table): the TTT-MLP layer of
the page's key designs ("TTT-MLP layer", "gate + bidirectional") with a linear
inner model f(u; W) = u W.  Independent references used: central finite
differences, torch's fp64 autograd, the delta-rule product form of the per-token
step, the exact geometric decay of the residual on a repeated token, an exact
rational-arithmetic step, the mini-batch dual form written with masked matrix
products, and invariants (teacher fixed point, causality, gate and
bidirectional wiring, state hand-off).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import ttt_linear_oracle as L

torch.set_default_dtype(torch.float64)


def _rng(seed):
    return np.random.default_rng(seed)


def _qkv(seed, T, d):
    g = _rng(seed)
    return [g.standard_normal((T, d)) for _ in range(3)]


def _torch_loss(W, k, v, loss):
    e = k @ W - v
    s = (e * e).sum()
    return s / e.shape[-1] if loss == "mean" else s


# ----------------------------------------------------------------------------
# the inner loss and its gradient
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("loss", ["mean", "sum"])
def test_grad_matches_central_differences(loss):
    d = 5
    g = _rng(1)
    W = g.standard_normal((d, d)) / 2
    k, v = g.standard_normal(d), g.standard_normal(d)
    an = L.linear_grad(W, k, v, loss)[0]
    h = 1e-6
    fd = np.zeros_like(W)
    for i in range(d):
        for j in range(d):
            Wp, Wm = W.copy(), W.copy()
            Wp[i, j] += h
            Wm[i, j] -= h
            fd[i, j] = (L.linear_loss(Wp, k, v, loss) - L.linear_loss(Wm, k, v, loss)) / (2 * h)
    np.testing.assert_allclose(an, fd, rtol=1e-7, atol=1e-8)


# ----------------------------------------------------------------------------
# the scan
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("loss", ["mean", "sum"])
def test_b1_equals_per_token_gradient_descent_autograd(loss):
    """b = 1: W_t = W_{t-1} - eta grad l(W_{t-1}; x_t) (torch autograd), z_t = q_t W_t."""
    T, d, eta = 12, 4, 0.07
    Q, K, V = _qkv(2, T, d)
    W0 = _rng(3).standard_normal((d, d)) / 2
    Z, WT = L.scan_head_linear(Q, K, V, W0, eta, 1, loss)
    w = torch.tensor(W0)
    for t in range(T):
        a = w.clone().requires_grad_()
        (gw,) = torch.autograd.grad(_torch_loss(a, torch.tensor(K[t]), torch.tensor(V[t]), loss), (a,))
        w = w - eta * gw
        np.testing.assert_allclose(Z[t], (torch.tensor(Q[t]) @ w).numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(WT, w.numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("b,T", [(4, 11), (3, 9), (16, 7)])
def test_minibatch_rule_autograd(b, T):
    """Within a mini-batch starting at W^B, token t reads out with W^B minus eta
    times the gradient of the summed losses of tokens s <= t, all taken at W^B."""
    d, eta = 3, 0.1
    Q, K, V = _qkv(4 + b, T, d)
    W0 = _rng(5).standard_normal((d, d))
    Z, WT = L.scan_head_linear(Q, K, V, W0, eta, b, "mean")
    w = torch.tensor(W0)
    for start in range(0, T, b):
        stop = min(start + b, T)
        for t in range(start, stop):
            a = w.clone().requires_grad_()
            tot = sum(_torch_loss(a, torch.tensor(K[s]), torch.tensor(V[s]), "mean") for s in range(start, t + 1))
            (gw,) = torch.autograd.grad(tot, (a,))
            st = w - eta * gw
            np.testing.assert_allclose(Z[t], (torch.tensor(Q[t]) @ st).numpy(), rtol=1e-11, atol=1e-12)
        w = st
    np.testing.assert_allclose(WT, w.numpy(), rtol=1e-11, atol=1e-12)


def test_b1_is_the_delta_rule():
    """Per token the step is W_t = (I - beta k^T k) W_{t-1} + beta k^T v with beta = eta c
    (c = 2/d): the delta rule, written here as a product and a rank-one correction."""
    T, d, eta = 20, 6, 0.3
    Q, K, V = _qkv(6, T, d)
    W0 = _rng(7).standard_normal((d, d)) / 3
    Z, WT = L.scan_head_linear(Q, K, V, W0, eta, 1, "mean")
    beta = eta * 2.0 / d
    W = W0.copy()
    for t in range(T):
        k, v = K[t][:, None], V[t][None, :]
        W = (np.eye(d) - beta * (k @ k.T)) @ W + beta * (k @ v)
        np.testing.assert_allclose(Z[t], Q[t] @ W, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(WT, W, rtol=1e-12, atol=1e-13)


def test_repeated_token_residual_decays_geometrically():
    """One token (k, v) seen T times with b = 1: the residual r_t = k W_t - v obeys
    r_t = (1 - eta c ||k||^2) r_{t-1} exactly, so r_T = (1 - eta c ||k||^2)^T r_0."""
    T, d, eta = 30, 8, 0.05
    g = _rng(8)
    k, v = g.standard_normal(d), g.standard_normal(d)
    W0 = g.standard_normal((d, d)) / 3
    K = np.tile(k, (T, 1))
    V = np.tile(v, (T, 1))
    Z, WT = L.scan_head_linear(K, K, V, W0, eta, 1, "mean")  # q = k: z_t = k W_t
    rho = 1.0 - eta * (2.0 / d) * float(k @ k)
    r0 = k @ W0 - v
    for t in range(T):
        np.testing.assert_allclose(Z[t] - v, rho ** (t + 1) * r0, rtol=1e-10, atol=1e-12)


def test_exact_step_in_rational_arithmetic():
    """d = 2, two tokens, b = 2 and b = 1: the definition worked out with exact fractions."""
    F = Fraction
    W0 = [[F(1), F(-1, 2)], [F(1, 4), F(2)]]
    K = [[F(1), F(2)], [F(-1), F(1, 2)]]
    V = [[F(3, 2), F(0)], [F(1), F(-1)]]
    Q = [[F(1, 2), F(1)], [F(2), F(-1)]]
    eta, c = F(1, 10), F(2, 2)  # mean loss: c = 2/d = 1

    def matvec(k, W):  # row vector times matrix
        return [sum(k[i] * W[i][j] for i in range(2)) for j in range(2)]

    def grad(W, k, v):  # k^T c (k W - v)
        gr = [c * (a - b) for a, b in zip(matvec(k, W), v)]
        return [[k[i] * gr[j] for j in range(2)] for i in range(2)]

    def sub(W, G):
        return [[W[i][j] - eta * G[i][j] for j in range(2)] for i in range(2)]

    f = lambda M: np.array([[float(x) for x in r] for r in M])
    # b = 2: both gradients at W0
    G0, G1 = grad(W0, K[0], V[0]), grad(W0, K[1], V[1])
    W_a = sub(W0, G0)
    W_b = sub(W_a, G1)
    Z, WT = L.scan_head_linear(f(Q), f(K), f(V), f(W0), 0.1, 2, "mean")
    np.testing.assert_allclose(Z[0], [float(x) for x in matvec(Q[0], W_a)], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(Z[1], [float(x) for x in matvec(Q[1], W_b)], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(WT, f(W_b), rtol=1e-15, atol=1e-15)
    # b = 1: the second gradient at the updated state
    W_c = sub(W_a, grad(W_a, K[1], V[1]))
    Z1, WT1 = L.scan_head_linear(f(Q), f(K), f(V), f(W0), 0.1, 1, "mean")
    np.testing.assert_allclose(Z1[1], [float(x) for x in matvec(Q[1], W_c)], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(WT1, f(W_c), rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("b,T", [(16, 50), (5, 23), (1, 7)])
def test_dual_form_equals_primal(b, T):
    """Mini-batch dual form: G = c (K W - V), Z = Q W - eta tril(Q K^T) G (diagonal
    included), W' = W - eta K^T G, with masked matrix products only."""
    d, eta = 8, 0.05
    Q, K, V = _qkv(9, T, d)
    W0 = _rng(10).standard_normal((d, d)) / 3
    Z, WT = L.scan_head_linear(Q, K, V, W0, eta, b, "mean")
    W = W0.copy()
    Zd = np.zeros_like(Z)
    for s in range(0, T, b):
        Kb, Vb, Qb = K[s:s + b], V[s:s + b], Q[s:s + b]
        G = (2.0 / d) * (Kb @ W - Vb)
        Zd[s:s + b] = Qb @ W - eta * np.tril(Qb @ Kb.T) @ G
        W = W - eta * Kb.T @ G
    np.testing.assert_allclose(Z, Zd, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(WT, W, rtol=1e-11, atol=1e-12)


def test_teacher_fixed_point_and_eta_zero():
    """v = k W* for every token and W_0 = W*: every gradient is zero, the state stays
    W* and z_t = q_t W*.  eta = 0: z_t = q_t W_0 whatever the targets."""
    T, d = 25, 6
    Q, K, _ = _qkv(11, T, d)
    Ws = _rng(12).standard_normal((d, d))
    Z, WT = L.scan_head_linear(Q, K, K @ Ws, Ws, 0.2, 4, "mean")
    np.testing.assert_allclose(Z, Q @ Ws, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(WT, Ws, rtol=1e-13, atol=1e-13)
    V = _rng(13).standard_normal((T, d))
    Z0, W0T = L.scan_head_linear(Q, K, V, Ws, 0.0, 4, "mean")
    np.testing.assert_allclose(Z0, Q @ Ws, rtol=1e-14, atol=1e-14)  # row-by-row vs matrix product order
    np.testing.assert_array_equal(W0T, Ws)


# ----------------------------------------------------------------------------
# the layer: projections, gate, directions
# ----------------------------------------------------------------------------

def _layer_problem(seed, T, H, d):
    g = _rng(seed)
    D = H * d
    X = g.standard_normal((T, D))
    theta = g.standard_normal((3, D, D)) / math.sqrt(D)
    W0 = g.standard_normal((H, d, d)) / math.sqrt(d)
    return X, theta, W0


def test_forward_is_causal_and_alpha_zero_is_identity():
    T, H, d = 40, 2, 4
    X, theta, W0 = _layer_problem(14, T, H, d)
    alpha = np.full(H * d, 0.3)
    a = L.ttt_linear_forward(X, theta, W0, alpha, eta=0.1, b=4)
    X2 = X.copy()
    X2[25:] += 1.0
    b = L.ttt_linear_forward(X2, theta, W0, alpha, eta=0.1, b=4)
    np.testing.assert_array_equal(a["Y"][:25], b["Y"][:25])  # tokens before 25 see no change
    assert not np.allclose(a["Y"][25:], b["Y"][25:])
    z = L.ttt_linear_forward(X, theta, W0, np.zeros(H * d), eta=0.1, b=4)
    np.testing.assert_array_equal(z["Y"], X)
    # gate wiring: y - x = tanh(alpha) z per channel
    np.testing.assert_allclose(a["Y"] - X, np.tanh(0.3) * a["Z"], rtol=1e-12, atol=1e-12)


def test_projection_per_head_and_state_hand_off():
    """Head h sees q = (X theta_Q^T)[:, h d:(h+1) d] (computed here by a plain matmul);
    continuing from the state after T1 tokens equals the whole run when T1 is a
    multiple of b."""
    T, H, d, b = 32, 3, 4, 4
    X, theta, W0 = _layer_problem(15, T, H, d)
    alpha = np.full(H * d, 0.2)
    full = L.ttt_linear_forward(X, theta, W0, alpha, eta=0.08, b=b)
    for h in range(H):
        sl = slice(h * d, (h + 1) * d)
        Q, K, V = [(X @ theta[p].T)[:, sl] for p in range(3)]
        Zh, _ = L.scan_head_linear(Q, K, V, W0[h], 0.08, b)
        np.testing.assert_allclose(full["Z"][:, sl], Zh, rtol=1e-12, atol=1e-12)
    T1 = 12
    first = L.ttt_linear_forward(X[:T1], theta, W0, alpha, eta=0.08, b=b)
    rest = L.ttt_linear_forward(X[T1:], theta, first["W_T"][0], alpha, eta=0.08, b=b)
    np.testing.assert_allclose(np.concatenate([first["Y"], rest["Y"]]), full["Y"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(rest["W_T"], full["W_T"], rtol=1e-12, atol=1e-12)


def test_bidir_composition_and_reverse_is_flip():
    T, H, d = 30, 2, 4
    X, theta, W0 = _layer_problem(16, T, H, d)
    af, ab = np.full(H * d, 0.1), np.full(H * d, -0.25)
    bd = L.ttt_linear_bidir(X, theta, W0, af, ab, eta=0.1, b=4)
    f = L.ttt_linear_forward(X, theta, W0, af, eta=0.1, b=4)
    r = L.ttt_linear_forward(f["Y"], theta, W0, ab, eta=0.1, b=4, reverse=True)
    np.testing.assert_array_equal(bd["Y"], r["Y"])
    np.testing.assert_array_equal(bd["Xp"], f["Y"])
    # the reversed pass equals the forward pass on the flipped sequence, flipped back
    rf = L.ttt_linear_forward(f["Y"][::-1], theta, W0, ab, eta=0.1, b=4)
    np.testing.assert_allclose(r["Y"], rf["Y"][::-1], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(r["Z"], rf["Z"][::-1], rtol=1e-13, atol=1e-13)


def test_workers_do_not_change_the_result():
    T, H, d = 20, 4, 4
    X, theta, W0 = _layer_problem(17, T, H, d)
    alpha = np.full(H * d, 0.1)
    a = L.ttt_linear_forward(X, theta, W0, alpha, eta=0.1, b=4, workers=1)
    b = L.ttt_linear_forward(X, theta, W0, alpha, eta=0.1, b=4, workers=3)
    np.testing.assert_array_equal(a["Y"], b["Y"])
