"""Pins of the backward oracle (oracle/ttt_backward_oracle.py) to things other
than itself: the forward oracle's values (an independent implementation of the
layer), central finite differences of the forward oracle, the closed form at
eta = 0, the gate's exact cases, causality, and the composition rules.
CPU only."""
import numpy as np
import pytest

from oracle import ttt_backward_oracle as BO
from oracle import ttt_oracle as O

NAMES = ["X", "theta", "W1_0", "W2_0", "alpha"]


def _case(seed, T=9, H=2, d=3, m=5, B=1, alpha_scale=0.7):
    rng = np.random.default_rng(seed)
    D = H * d
    return dict(
        X=rng.normal(size=(B, T, D)),
        theta=rng.normal(size=(3, D, D)) / np.sqrt(D),
        W1_0=rng.normal(size=(H, d, m)) / np.sqrt(d),
        W2_0=rng.normal(size=(H, m, d)) / np.sqrt(m),
        alpha=rng.normal(size=D) * alpha_scale,
        dY=rng.normal(size=(B, T, D)),
    )


def _direction(rng, x):
    """A random direction with the input's own scale (rms), so that steps are relative."""
    u = rng.normal(size=x.shape)
    return u * max(float(np.sqrt(np.mean(x * x))), 1e-3)


def _richardson(L, c, name, u, h=1e-4):
    """Central difference of L along u, Richardson-extrapolated: (4 D(h/2) - D(h)) / 3
    cancels the h^2 term, leaving O(h^4)."""
    def D(e):
        cp, cm = dict(c), dict(c)
        cp[name] = c[name] + e * u
        cm[name] = c[name] - e * u
        return (L(cp) - L(cm)) / (2 * e)
    return (4 * D(h / 2) - D(h)) / 3


def _fwd(c, **kw):
    return O.ttt_forward(c["X"], c["theta"], c["W1_0"], c["W2_0"], c["alpha"], **kw)["Y"]


def _bwd(c, **kw):
    return BO.ttt_mlp_backward(c["X"], c["theta"], c["W1_0"], c["W2_0"], c["alpha"], c["dY"], **kw)


@pytest.mark.parametrize("b,reverse,loss,form", [(1, False, "mean", "erf"), (4, False, "mean", "erf"),
                                                 (4, True, "sum", "erf"), (3, False, "mean", "tanh")])
def test_torch_forward_equals_numpy_oracle(b, reverse, loss, form):
    c = _case(1, T=10)
    kw = dict(eta=0.3, b=b, reverse=reverse, loss=loss)
    y_np = O.ttt_forward(c["X"], c["theta"], c["W1_0"], c["W2_0"], c["alpha"], gelu_form=form, **kw)["Y"]
    y_t = BO.layer_forward(c["X"], c["theta"], c["W1_0"], c["W2_0"], c["alpha"], gelu_form=form, **kw)
    np.testing.assert_allclose(y_t, y_np, rtol=0, atol=1e-12)


@pytest.mark.parametrize("b,reverse,loss,form", [(1, False, "mean", "erf"), (4, False, "mean", "erf"),
                                                 (4, True, "sum", "erf"), (3, True, "mean", "tanh")])
def test_central_differences_of_the_forward_oracle(b, reverse, loss, form):
    """<grad, u> against (L(p + eps u) - L(p - eps u)) / (2 eps), L = sum(dY * Y) of
    the NumPy forward oracle, for a random direction u in each input."""
    c = _case(2, T=10)
    kw = dict(eta=0.3, b=b, reverse=reverse, loss=loss, gelu_form=form)
    g = _bwd(c, **kw)
    rng = np.random.default_rng(7)
    for name, gname in zip(NAMES, ["dX", "dtheta", "dW1_0", "dW2_0", "dalpha"]):
        u = _direction(rng, c[name])
        fd = _richardson(lambda cc: np.sum(cc["dY"] * _fwd(cc, **kw)), c, name, u)
        an = float(np.sum(g[gname] * u))
        assert abs(fd - an) <= 1e-8 * max(1.0, abs(fd)), (name, fd, an)


def test_central_differences_bidirectional():
    c = _case(3, T=8)
    c["alpha_b"] = np.random.default_rng(4).normal(size=c["alpha"].shape) * 0.7
    kw = dict(eta=0.3, b=3, loss="mean", gelu_form="erf")
    g = BO.ttt_mlp_bidir_backward(c["X"], c["theta"], c["W1_0"], c["W2_0"], c["alpha"], c["alpha_b"], c["dY"], **kw)

    def L(cc):
        y = O.ttt_bidir(cc["X"], cc["theta"], cc["W1_0"], cc["W2_0"], cc["alpha"], cc["alpha_b"], **kw)["Y"]
        return np.sum(cc["dY"] * y)

    rng = np.random.default_rng(9)
    for name, gname in [("X", "dX"), ("theta", "dtheta"), ("W1_0", "dW1_0"), ("W2_0", "dW2_0"),
                        ("alpha", "dalpha_f"), ("alpha_b", "dalpha_b")]:
        u = _direction(rng, c[name])
        fd = _richardson(L, c, name, u)
        an = float(np.sum(g[gname] * u))
        assert abs(fd - an) <= 1e-8 * max(1.0, abs(fd)), (name, fd, an)


def _gelu_grad(a):
    return O.gelu_grad(a, "erf")


def test_eta_zero_closed_form():
    """eta = 0: the state never moves, so per head Z = GELU(X theta_Q^T W1) W2 and
    the gradients have a closed form (K and V do not enter)."""
    c = _case(5, T=7, H=2, d=3, m=4)
    g = _bwd(c, eta=0.0, b=2)
    X, th, W1, W2, al, dY = (c[k][0] if k in ("X", "dY") else c[k] for k in ["X", "theta", "W1_0", "W2_0",
                                                                            "alpha", "dY"])
    H, d, m = W1.shape
    tg = np.tanh(al)
    dX = dY.copy()
    dth = np.zeros_like(th)
    dW1 = np.zeros_like(W1)
    dW2 = np.zeros_like(W2)
    dal = np.zeros_like(al)
    for h in range(H):
        sl = slice(h * d, (h + 1) * d)
        Q = X @ th[0, sl].T
        Aq = Q @ W1[h]
        Hq = O.gelu(Aq)
        Z = Hq @ W2[h]
        dZ = tg[sl] * dY[:, sl]
        dal[sl] = np.sum(dY[:, sl] * Z, axis=0) * (1 - tg[sl] ** 2)
        dW2[h] = Hq.T @ dZ
        dAq = (dZ @ W2[h].T) * _gelu_grad(Aq)
        dW1[h] = Q.T @ dAq
        dQ = dAq @ W1[h].T
        dth[0, sl] = dQ.T @ X
        dX += dQ @ th[0, sl]
    for got, want in [(g["dX"][0], dX), (g["dtheta"], dth), (g["dW1_0"], dW1), (g["dW2_0"], dW2),
                      (g["dalpha"], dal)]:
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_zero_gate():
    """alpha = 0: Y = X, so dX = dY exactly, theta and W_0 get nothing, and
    dalpha = sum_t dY * Z (tanh'(0) = 1)."""
    c = _case(6, T=9)
    c["alpha"] = np.zeros_like(c["alpha"])
    kw = dict(eta=0.3, b=4)
    g = _bwd(c, **kw)
    assert np.array_equal(g["dX"], c["dY"])
    for k in ["dtheta", "dW1_0", "dW2_0"]:
        assert not np.any(g[k]), k
    Z = O.ttt_forward(c["X"], c["theta"], c["W1_0"], c["W2_0"], c["alpha"], **kw)["Z"]
    np.testing.assert_allclose(g["dalpha"], np.sum(c["dY"] * Z, axis=(0, 1)), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("reverse", [False, True])
def test_causality(reverse):
    """With dY on one token only, the forward pass's dX vanishes after it (the
    reversed pass's before it): outputs depend only on tokens already scanned."""
    c = _case(8, T=12)
    P = 6
    c["dY"][:, :P] = 0.0
    c["dY"][:, P + 1:] = 0.0
    g = _bwd(c, eta=0.3, b=4, reverse=reverse)
    after = g["dX"][:, :P] if reverse else g["dX"][:, P + 1:]
    before = g["dX"][:, P + 1:] if reverse else g["dX"][:, :P]
    assert not np.any(after)
    assert np.any(before)


def test_head_subset_and_batch():
    """Heads are independent, and sequences are independent with shared theta and
    W_0: restricting to heads whose channels carry dY changes nothing, and a
    batch's gradients are the per-sequence gradients (dX) or their sums."""
    c = _case(10, T=8, H=3, B=2)
    c["dY"][..., 3:6] = 0.0  # head 1 carries no gradient
    kw = dict(eta=0.3, b=3)
    full = _bwd(c, **kw)
    sub = _bwd(c, heads=[0, 2], **kw)
    for k in full:
        np.testing.assert_allclose(sub[k], full[k], rtol=1e-13, atol=1e-13)
    parts = [_bwd(dict(c, X=c["X"][i:i + 1], dY=c["dY"][i:i + 1]), **kw) for i in range(2)]
    np.testing.assert_allclose(full["dX"], np.concatenate([p["dX"] for p in parts]), rtol=1e-13, atol=1e-13)
    for k in ["dtheta", "dW1_0", "dW2_0", "dalpha"]:
        np.testing.assert_allclose(full[k], parts[0][k] + parts[1][k], rtol=1e-12, atol=1e-13)
    with pytest.raises(ValueError):
        _bwd(c, heads=[0], **kw)


def test_bidirectional_chain_rule():
    """The bidirectional gradients chain the two directions: the reversed pass's
    dX is the forward pass's dY; theta and W_0 collect both directions."""
    c = _case(11, T=8)
    ab = np.random.default_rng(12).normal(size=c["alpha"].shape) * 0.7
    kw = dict(eta=0.3, b=3)
    g = BO.ttt_mlp_bidir_backward(c["X"], c["theta"], c["W1_0"], c["W2_0"], c["alpha"], ab, c["dY"], **kw)
    Xp = O.ttt_forward(c["X"], c["theta"], c["W1_0"], c["W2_0"], c["alpha"], **kw)["Y"]
    r = BO.ttt_mlp_backward(Xp, c["theta"], c["W1_0"], c["W2_0"], ab, c["dY"], reverse=True, **kw)
    f = BO.ttt_mlp_backward(c["X"], c["theta"], c["W1_0"], c["W2_0"], c["alpha"], r["dX"], **kw)
    np.testing.assert_allclose(g["dX"], f["dX"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dalpha_f"], f["dalpha"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dalpha_b"], r["dalpha"], rtol=1e-11, atol=1e-12)
    for k in ["dtheta", "dW1_0", "dW2_0"]:
        np.testing.assert_allclose(g[k], f[k] + r[k], rtol=1e-11, atol=1e-12)


def test_empty_sequence():
    c = _case(13, T=0)
    g = _bwd(c, eta=0.3, b=4)
    assert g["dX"].shape == c["X"].shape
    for k in ["dtheta", "dW1_0", "dW2_0", "dalpha"]:
        assert not np.any(g[k])
