"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names the part of the method it pins ("One-Minute Video Generation
with Test-Time Training", paper-notes page, key designs: "TTT-MLP layer" for
the inner model, loss, update and read-out; "gate + bidirectional" for the
gate and the two directions).  Independent references used: textbook values
of the normal CDF, mpmath at 40 digits, central finite differences, torch's
fp64 autograd and GELU, closed forms of special cases, and invariants
(symmetry, causality, fixed points, state hand-off).
"""
import math
import os

import mpmath
import numpy as np
import pytest
import torch

from oracle import ttt_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
torch.set_default_dtype(torch.float64)


def _rng(seed):
    return np.random.default_rng(seed)


def _small_problem(seed, T, H, d, m, x_scale=1.0):
    g = _rng(seed)
    D = H * d
    X = g.standard_normal((T, D)) * x_scale
    theta = g.standard_normal((3, D, D)) / math.sqrt(D)
    W1 = g.standard_normal((H, d, m)) / math.sqrt(d)
    W2 = g.standard_normal((H, m, d)) / math.sqrt(m)
    return X, theta, W1, W2


# ----------------------------------------------------------------------------
# GELU (inner model nonlinearity)
# ----------------------------------------------------------------------------

def test_gelu_matches_printed_normal_cdf_table():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "normal_cdf.txt")) if l.strip() and not l.startswith("#")]
    for xs, ps in rows:
        x, p = float(xs), float(ps)
        assert abs(O.gelu(x) - x * p) <= 1e-10 * max(1.0, abs(x))
        if x != 0.0:
            # Phi(x) recovered from GELU(x)/x
            assert abs(O.gelu(x) / x - p) <= 6e-11
    assert O.gelu_grad(0.0) == 0.5


def test_gelu_and_derivative_match_mpmath():
    xs = np.linspace(-6, 6, 121)
    for x in xs:
        xm = mpmath.mpf(float(x))
        g = xm * mpmath.ncdf(xm)
        dg = mpmath.diff(lambda t: t * mpmath.ncdf(t), xm)
        assert abs(O.gelu(x) - float(g)) <= 1e-15 * max(1, abs(x))
        assert abs(O.gelu_grad(x) - float(dg)) <= 1e-14
    for x in xs:
        xm = mpmath.mpf(float(x))
        f = lambda t: t / 2 * (1 + mpmath.tanh(mpmath.sqrt(2 / mpmath.pi) * (t + mpmath.mpf("0.044715") * t ** 3)))
        assert abs(O.gelu(x, "tanh") - float(f(xm))) <= 1e-15 * max(1, abs(x))
        assert abs(O.gelu_grad(x, "tanh") - float(mpmath.diff(f, xm))) <= 1e-14


def test_gelu_matches_torch_both_forms():
    a = torch.linspace(-8, 8, 1001, requires_grad=True)
    for form, approx in (("erf", "none"), ("tanh", "tanh")):
        y = torch.nn.functional.gelu(a, approximate=approx)
        (gy,) = torch.autograd.grad(y.sum(), a)
        np.testing.assert_allclose(O.gelu(a.detach().numpy(), form), y.detach().numpy(), rtol=0, atol=1e-15)
        np.testing.assert_allclose(O.gelu_grad(a.detach().numpy(), form), gy.numpy(), rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------
# loss and its gradient
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("d", [1, 2, 4])
@pytest.mark.parametrize("loss", ["mean", "sum"])
@pytest.mark.parametrize("form", ["erf", "tanh"])
def test_inner_grad_central_differences(d, loss, form):
    m = 4 * d
    g = _rng(100 + d)
    W1 = g.standard_normal((d, m)) / math.sqrt(d)
    W2 = g.standard_normal((m, d)) / math.sqrt(m)
    k = g.standard_normal(d)
    v = g.standard_normal(d)
    dW1, dW2 = O.inner_grad(W1, W2, k, v, loss, form)
    h = 1e-6
    for W, dW in ((W1, dW1[0]), (W2, dW2[0])):
        fd = np.zeros_like(W)
        for idx in np.ndindex(W.shape):
            old = W[idx]
            W[idx] = old + h
            lp = O.inner_loss(W1, W2, k, v, loss, form)
            W[idx] = old - h
            lm = O.inner_loss(W1, W2, k, v, loss, form)
            W[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        err = np.linalg.norm(fd - dW) / max(np.linalg.norm(dW), 1e-12)
        assert err < 1e-6, err


@pytest.mark.parametrize("loss", ["mean", "sum"])
def test_inner_grad_matches_torch_autograd(loss):
    d, m, n = 8, 32, 5
    g = _rng(7)
    W1 = g.standard_normal((d, m)) / math.sqrt(d)
    W2 = g.standard_normal((m, d)) / math.sqrt(m)
    K = g.standard_normal((n, d))
    V = g.standard_normal((n, d))
    dW1, dW2 = O.inner_grad(W1, W2, K, V, loss)
    for s in range(n):
        w1 = torch.tensor(W1, requires_grad=True)
        w2 = torch.tensor(W2, requires_grad=True)
        e = torch.nn.functional.gelu(torch.tensor(K[s]) @ w1) @ w2 - torch.tensor(V[s])
        l = (e * e).mean() if loss == "mean" else (e * e).sum()
        g1, g2 = torch.autograd.grad(l, (w1, w2))
        np.testing.assert_allclose(dW1[s], g1.numpy(), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dW2[s], g2.numpy(), rtol=1e-12, atol=1e-14)
        assert abs(O.inner_loss(W1, W2, K[s], V[s], loss) - l.item()) <= 1e-13 * max(1, l.item())


def test_loss_closed_forms():
    d, m = 4, 16
    g = _rng(3)
    W1 = g.standard_normal((d, m))
    k, v = g.standard_normal(d), g.standard_normal(d)
    # W2 = 0: f == 0, so the loss is the mean (or sum) of v^2
    assert abs(O.inner_loss(W1, np.zeros((m, d)), k, v, "mean") - np.mean(v * v)) < 1e-15
    assert abs(O.inner_loss(W1, np.zeros((m, d)), k, v, "sum") - np.sum(v * v)) < 1e-14
    # an exact fit has zero loss and zero gradient
    W2 = g.standard_normal((m, d))
    v_fit = O.mlp(k, W1, W2)
    assert O.inner_loss(W1, W2, k, v_fit) == 0.0
    dW1, dW2 = O.inner_grad(W1, W2, k, v_fit)
    assert np.abs(dW1).max() == 0.0 and np.abs(dW2).max() == 0.0


# ----------------------------------------------------------------------------
# one step, written out in 40-digit arithmetic
# ----------------------------------------------------------------------------

def test_single_token_step_by_hand_mpmath():
    mpmath.mp.dps = 40
    d, m, eta = 1, 4, 0.3
    w1 = [0.7, -1.1, 0.4, 2.0]  # W1 is 1 x 4
    w2 = [0.5, 0.25, -0.8, 0.1]  # W2 is 4 x 1
    k, v, q = 0.9, -0.35, 1.3
    M = mpmath.mpf
    gel = lambda a: a * mpmath.ncdf(a)
    dgel = lambda a: mpmath.ncdf(a) + a * mpmath.npdf(a)
    a = [M(k) * M(w) for w in w1]
    h = [gel(x) for x in a]
    e = sum(hi * M(w) for hi, w in zip(h, w2)) - M(v)
    g2 = 2 * e  # d = 1: mean and sum agree
    g1 = [g2 * M(w) * dgel(x) for w, x in zip(w2, a)]
    w1n = [M(w) - M(eta) * M(k) * gi for w, gi in zip(w1, g1)]
    w2n = [M(w) - M(eta) * hi * g2 for w, hi in zip(w2, h)]
    z = sum(gel(M(q) * w) * w2i for w, w2i in zip(w1n, w2n))
    Z, W1T, W2T = O.scan_head(np.array([[q]]), np.array([[k]]), np.array([[v]]),
                              np.array([w1]), np.array(w2)[:, None], eta, 1)
    assert abs(Z[0, 0] - float(z)) < 1e-15
    np.testing.assert_allclose(W1T[0], [float(x) for x in w1n], rtol=0, atol=1e-15)
    np.testing.assert_allclose(W2T[:, 0], [float(x) for x in w2n], rtol=0, atol=1e-15)
    mpmath.mp.dps = 15


# ----------------------------------------------------------------------------
# the scan: per-token rule, mini-batch rule, dual form
# ----------------------------------------------------------------------------

def _torch_loss(w1, w2, k, v, loss):
    e = torch.nn.functional.gelu(k @ w1) @ w2 - v
    return (e * e).mean() if loss == "mean" else (e * e).sum()


def test_b1_equals_per_token_gradient_descent_autograd():
    """b = 1: W_t = W_{t-1} - eta grad l(W_{t-1}; x_t), z_t = f(q_t; W_t)."""
    T, d, m, eta = 9, 4, 16, 0.2
    g = _rng(11)
    Q, K, V = (g.standard_normal((T, d)) for _ in range(3))
    W1 = g.standard_normal((d, m)) / 2
    W2 = g.standard_normal((m, d)) / 4
    Z, W1T, W2T = O.scan_head(Q, K, V, W1, W2, eta, 1)
    w1, w2 = torch.tensor(W1), torch.tensor(W2)
    for t in range(T):
        a1, a2 = w1.clone().requires_grad_(), w2.clone().requires_grad_()
        g1, g2 = torch.autograd.grad(_torch_loss(a1, a2, torch.tensor(K[t]), torch.tensor(V[t]), "mean"), (a1, a2))
        w1, w2 = w1 - eta * g1, w2 - eta * g2
        z = torch.nn.functional.gelu(torch.tensor(Q[t]) @ w1) @ w2
        np.testing.assert_allclose(Z[t], z.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(W1T, w1.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(W2T, w2.numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("b,T", [(4, 11), (3, 9), (8, 5)])
def test_minibatch_rule_autograd(b, T):
    """Within a mini-batch starting at W^B, token t reads out with
    W^B - eta * grad of the summed losses of the tokens s <= t, all at W^B."""
    d, m, eta = 3, 12, 0.15
    g = _rng(20 + b)
    Q, K, V = (g.standard_normal((T, d)) for _ in range(3))
    W1 = g.standard_normal((d, m)) / 2
    W2 = g.standard_normal((m, d)) / 3
    Z, W1T, W2T = O.scan_head(Q, K, V, W1, W2, eta, b, loss="sum")
    w1, w2 = torch.tensor(W1), torch.tensor(W2)
    for start in range(0, T, b):
        stop = min(start + b, T)
        for t in range(start, stop):
            a1, a2 = w1.clone().requires_grad_(), w2.clone().requires_grad_()
            tot = sum(_torch_loss(a1, a2, torch.tensor(K[s]), torch.tensor(V[s]), "sum") for s in range(start, t + 1))
            g1, g2 = torch.autograd.grad(tot, (a1, a2))
            s1, s2 = w1 - eta * g1, w2 - eta * g2
            z = torch.nn.functional.gelu(torch.tensor(Q[t]) @ s1) @ s2
            np.testing.assert_allclose(Z[t], z.numpy(), rtol=1e-11, atol=1e-12)
        w1, w2 = s1, s2
    np.testing.assert_allclose(W1T, w1.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(W2T, w2.numpy(), rtol=1e-11, atol=1e-12)


def _dual_form_head(Q, K, V, W1, W2, eta, b, loss="mean"):
    """The mini-batch scan rewritten without materialising W_t per token:
    Aq = Q W1 - eta tril(Q K^T) G1, Z = GELU(Aq) W2 - eta tril(GELU(Aq) Hk^T) G2."""
    T, d = Q.shape
    c = 2.0 / d if loss == "mean" else 2.0
    W1, W2 = W1.copy(), W2.copy()
    Z = np.zeros((T, d))
    for s0 in range(0, T, b):
        s1 = min(s0 + b, T)
        k, q, v = K[s0:s1], Q[s0:s1], V[s0:s1]
        A = k @ W1
        Hk = O.gelu(A)
        G2 = c * (Hk @ W2 - v)
        G1 = (G2 @ W2.T) * O.gelu_grad(A)
        Aq = q @ W1 - eta * np.tril(q @ k.T) @ G1
        Hq = O.gelu(Aq)
        Z[s0:s1] = Hq @ W2 - eta * np.tril(Hq @ Hk.T) @ G2
        W1 -= eta * k.T @ G1
        W2 -= eta * Hk.T @ G2
    return Z, W1, W2


@pytest.mark.parametrize("b,T", [(1, 13), (8, 37), (16, 50)])
def test_dual_form_equals_primal(b, T):
    d, m, eta = 8, 32, 0.05
    g = _rng(30 + b)
    Q, K, V = (g.standard_normal((T, d)) for _ in range(3))
    W1 = g.standard_normal((d, m)) / math.sqrt(d)
    W2 = g.standard_normal((m, d)) / math.sqrt(m)
    Zp, a1, a2 = O.scan_head(Q, K, V, W1, W2, eta, b)
    Zd, b1, b2 = _dual_form_head(Q, K, V, W1, W2, eta, b)
    np.testing.assert_allclose(Zp, Zd, rtol=0, atol=1e-12)
    np.testing.assert_allclose(a1, b1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(a2, b2, rtol=0, atol=1e-12)


def test_mean_loss_is_sum_loss_with_eta_over_d():
    """(1/d)||e||^2 with rate eta is ||e||^2 with rate eta/d; bitwise for d = 2^k."""
    T, d, m = 20, 8, 32
    g = _rng(5)
    Q, K, V = (g.standard_normal((T, d)) for _ in range(3))
    W1 = g.standard_normal((d, m)) / math.sqrt(d)
    W2 = g.standard_normal((m, d)) / math.sqrt(m)
    a = O.scan_head(Q, K, V, W1, W2, 0.1, 4, loss="mean")
    s = O.scan_head(Q, K, V, W1, W2, 0.1 / d, 4, loss="sum")
    for x, y in zip(a, s):
        assert np.array_equal(x, y)


def test_gradient_descent_reduces_loss_on_a_repeated_token():
    d, m, eta = 4, 16, 0.05
    g = _rng(9)
    W1 = g.standard_normal((d, m)) / 2
    W2 = g.standard_normal((m, d)) / 4
    k, v = g.standard_normal(d), g.standard_normal(d)
    T = 400
    K = np.tile(k, (T, 1))
    V = np.tile(v, (T, 1))
    losses = []
    w1, w2 = W1, W2
    for t in range(T):
        losses.append(O.inner_loss(w1, w2, k, v))
        _, w1, w2 = O.scan_head(K[t:t + 1], K[t:t + 1], V[t:t + 1], w1, w2, eta, 1)
    assert all(b <= a + 1e-15 for a, b in zip(losses, losses[1:]))
    assert losses[-1] < 1e-3 * losses[0]


def test_teacher_state_is_a_fixed_point():
    """If every v_t = f(k_t; W*) and the scan starts at W*, the state never moves
    and z_t = f(q_t; W*)."""
    T, d, m = 24, 4, 16
    g = _rng(12)
    Q, K = g.standard_normal((T, d)), g.standard_normal((T, d))
    W1 = g.standard_normal((d, m)) / 2
    W2 = g.standard_normal((m, d)) / 4
    V = O.mlp(K, W1, W2)
    Z, a1, a2 = O.scan_head(Q, K, V, W1, W2, 0.3, 4)
    np.testing.assert_allclose(a1, W1, rtol=0, atol=1e-15)
    np.testing.assert_allclose(a2, W2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(Z, O.mlp(Q, W1, W2), rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------
# projections, head split and gate
# ----------------------------------------------------------------------------

def test_projection_orientation_one_hot_tokens():
    H, d = 3, 4
    D = H * d
    g = _rng(1)
    theta = g.standard_normal((3, D, D))
    X = np.eye(D)  # token i is the unit vector e_i
    Qh, Kh, Vh = O.project(X, theta, H)
    for p, P in enumerate((Qh, Kh, Vh)):
        for h in range(H):
            for i in range(D):
                # theta is [out, in]: channel j of token e_i is theta[p][j, i]
                np.testing.assert_array_equal(P[h, i], theta[p][h * d:(h + 1) * d, i])


def test_eta_zero_is_a_plain_mlp_and_gate_wiring():
    """eta = 0: the state stays W_0 and z_t = GELU(q_t W1_0) W2_0 per head;
    Y = X + tanh(alpha) z (checked with torch matmul/GELU)."""
    T, H, d, m = 10, 3, 4, 16
    X, theta, W1, W2 = _small_problem(2, T, H, d, m)
    alpha = np.linspace(-0.5, 0.5, H * d)
    r = O.ttt_forward(X, theta, W1, W2, alpha, eta=0.0, b=4)
    Xt, th = torch.tensor(X), torch.tensor(theta)
    Q, K, V = (Xt @ th[p].T for p in range(3))
    Z = torch.cat([torch.nn.functional.gelu(Q[:, h * d:(h + 1) * d] @ torch.tensor(W1[h])) @ torch.tensor(W2[h])
                   for h in range(H)], dim=1)
    np.testing.assert_allclose(r["Z"], Z.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["Y"], (Xt + torch.tanh(torch.tensor(alpha)) * Z).numpy(), rtol=0, atol=1e-13)
    np.testing.assert_array_equal(r["W1_T"][0], W1)
    np.testing.assert_array_equal(r["W2_T"][0], W2)


def test_gate_alpha_zero_and_saturated():
    T, H, d, m = 12, 2, 4, 16
    X, theta, W1, W2 = _small_problem(4, T, H, d, m)
    r0 = O.ttt_forward(X, theta, W1, W2, np.zeros(H * d), eta=0.1, b=4)
    assert np.array_equal(r0["Y"], X)
    r1 = O.ttt_forward(X, theta, W1, W2, np.full(H * d, 40.0), eta=0.1, b=4)
    assert np.array_equal(r1["Y"], X + r1["Z"])  # tanh(40) == 1 in fp64
    assert np.array_equal(r0["Z"], r1["Z"])


# ----------------------------------------------------------------------------
# directions
# ----------------------------------------------------------------------------

def test_forward_is_causal():
    """Outputs at tokens < t0 depend only on tokens < t0."""
    T, H, d, m = 20, 2, 4, 16
    X, theta, W1, W2 = _small_problem(6, T, H, d, m)
    a = O.ttt_forward(X, theta, W1, W2, np.full(H * d, 0.1), eta=0.1, b=4)
    X2 = X.copy()
    X2[13:] = _rng(99).standard_normal(X2[13:].shape)
    b = O.ttt_forward(X2, theta, W1, W2, np.full(H * d, 0.1), eta=0.1, b=4)
    np.testing.assert_array_equal(a["Z"][:13], b["Z"][:13])
    assert not np.allclose(a["Z"][13:], b["Z"][13:])


def test_reverse_pass_is_anticausal_with_batches_cut_from_the_end():
    """Reversed pass: outputs at tokens >= t0 depend only on tokens >= t0, when
    T - t0 is a multiple of b (mini-batches are cut from the reversed start)."""
    T, H, d, m, b = 22, 2, 4, 16, 4
    X, theta, W1, W2 = _small_problem(7, T, H, d, m)
    alpha = np.full(H * d, 0.1)
    full = O.ttt_forward(X, theta, W1, W2, alpha, eta=0.1, b=b, reverse=True)
    t0 = T - 12
    tail = O.ttt_forward(X[t0:], theta, W1, W2, alpha, eta=0.1, b=b, reverse=True)
    np.testing.assert_allclose(full["Z"][t0:], tail["Z"], rtol=0, atol=1e-14)
    # the reversed pass is the forward pass on the flipped sequence
    fl = O.ttt_forward(X[::-1], theta, W1, W2, alpha, eta=0.1, b=b)
    np.testing.assert_array_equal(full["Z"], fl["Z"][::-1])
    np.testing.assert_array_equal(full["Y"], fl["Y"][::-1])
    np.testing.assert_array_equal(full["W1_T"], fl["W1_T"])


def test_bidir_composition_and_gate_separation():
    T, H, d, m = 16, 2, 4, 16
    X, theta, W1, W2 = _small_problem(8, T, H, d, m)
    af, ab = np.full(H * d, 0.1), np.full(H * d, 0.2)
    r = O.ttt_bidir(X, theta, W1, W2, af, ab, eta=0.1, b=4)
    # alpha_b = 0: the output is the forward pass's output
    r0 = O.ttt_bidir(X, theta, W1, W2, af, np.zeros(H * d), eta=0.1, b=4)
    f = O.ttt_forward(X, theta, W1, W2, af, eta=0.1, b=4)
    np.testing.assert_array_equal(r0["Y"], f["Y"])
    np.testing.assert_array_equal(r["Xp"], f["Y"])
    # alpha_f = 0: X' = X, so the output is the reversed pass on X with alpha_b
    r1 = O.ttt_bidir(X, theta, W1, W2, np.zeros(H * d), ab, eta=0.1, b=4)
    rv = O.ttt_forward(X, theta, W1, W2, ab, eta=0.1, b=4, reverse=True)
    np.testing.assert_array_equal(r1["Y"], rv["Y"])
    # swapped gates give a different result
    rs = O.ttt_bidir(X, theta, W1, W2, ab, af, eta=0.1, b=4)
    assert not np.allclose(rs["Y"], r["Y"])


def test_state_handoff_between_chunks():
    """forward(X[:T1]) -> W_T1; continuing from W_T1 over X[T1:] equals forward(X)[T1:]."""
    T, T1, d, m, b = 40, 24, 4, 16, 8
    g = _rng(13)
    Q, K, V = (g.standard_normal((T, d)) for _ in range(3))
    W1 = g.standard_normal((d, m)) / 2
    W2 = g.standard_normal((m, d)) / 4
    Z, a1, a2 = O.scan_head(Q, K, V, W1, W2, 0.1, b)
    Za, m1, m2 = O.scan_head(Q[:T1], K[:T1], V[:T1], W1, W2, 0.1, b)
    Zb, c1, c2 = O.scan_head(Q[T1:], K[T1:], V[T1:], m1, m2, 0.1, b)
    np.testing.assert_array_equal(np.concatenate([Za, Zb]), Z)
    np.testing.assert_array_equal(c1, a1)
    np.testing.assert_array_equal(c2, a2)


def test_empty_sequence_and_batch_of_sequences():
    H, d, m = 2, 4, 16
    _, theta, W1, W2 = _small_problem(14, 1, H, d, m)
    r = O.ttt_forward(np.zeros((1, 0, H * d)), theta, W1, W2, np.full(H * d, 0.1), eta=0.1, b=4)
    assert r["Y"].shape == (1, 0, H * d)
    np.testing.assert_array_equal(r["W1_T"][0], W1)
    g = _rng(15)
    X = g.standard_normal((3, 9, H * d))
    rb = O.ttt_forward(X, theta, W1, W2, np.full(H * d, 0.1), eta=0.1, b=4)
    for s in range(3):
        rs = O.ttt_forward(X[s], theta, W1, W2, np.full(H * d, 0.1), eta=0.1, b=4)
        np.testing.assert_array_equal(rb["Y"][s], rs["Y"])


def test_head_subset_matches_full_layer():
    T, H, d, m = 14, 4, 4, 16
    X, theta, W1, W2 = _small_problem(16, T, H, d, m)
    alpha = np.linspace(0, 1, H * d)
    full = O.ttt_forward(X, theta, W1, W2, alpha, eta=0.1, b=4, reverse=True)
    sub = O.ttt_forward(X, theta, W1, W2, alpha, eta=0.1, b=4, reverse=True, heads=[3, 1])
    cols = np.r_[12:16, 4:8]
    np.testing.assert_allclose(sub["Z"], full["Z"][:, cols], rtol=0, atol=1e-14)
    np.testing.assert_allclose(sub["Y"], full["Y"][:, cols], rtol=0, atol=1e-14)
    np.testing.assert_array_equal(sub["W1_T"][0, 0], full["W1_T"][0, 3])
