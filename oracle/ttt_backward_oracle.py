"""Plain fp64 CPU oracle of the TTT-MLP layer's backward (test infrastructure only).

Like ttt_oracle, this module is the checker, not the product: only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it.  It shares
no code with the HIP library.

What it computes: the outer-loop gradients of the layer of "One-Minute Video
Generation with Test-Time Training" (paper-notes page, key designs "TTT-MLP
layer" and "gate + bidirectional"; the page's training section trains theta_K,
theta_V, theta_Q, the initial state and the gate with the rest of the model).
For an upstream gradient dY of the layer output Y, it returns the
vector-Jacobian products

    dX = (dY . dY/dX),  dtheta,  dW1_0,  dW2_0,  dalpha (dalpha_f, dalpha_b)

that is, the gradients of the scalar L = sum(dY * Y) with respect to each
input.  The forward function is the same layer as ttt_oracle's, written
again in float64 torch so that it can be differentiated, and in the plainest
form of the definition: every token's inner step is taken with torch's own
gradient of the inner loss l(W; x_s) = ||f(k_s; W) - v_s||^2 at the state
its mini-batch starts from (no hand-derived inner gradient), the state of
every token is materialised (primal form), and torch's autograd
differentiates the whole recurrence, inner gradients included.  The readings
of ttt_oracle's header hold unchanged (mean loss by default, erf GELU, theta
[out, in], mini-batches, sequential bidirectional composition with X' kept
in float64).

Slow by design: one autograd call per token and head.  Meant for the small
cases of the tests and for prefixes of the full-size workloads.
"""
from __future__ import annotations

import math

import numpy as np
import torch

__all__ = ["layer_forward", "ttt_mlp_backward", "ttt_mlp_bidir_backward"]

_INV_SQRT2 = 1.0 / math.sqrt(2.0)
_TANH_C = math.sqrt(2.0 / math.pi)
_TANH_K = 0.044715


def _gelu(a, form):
    if form == "erf":
        return 0.5 * a * (1.0 + torch.erf(a * _INV_SQRT2))
    if form == "tanh":
        return 0.5 * a * (1.0 + torch.tanh(_TANH_C * (a + _TANH_K * a ** 3)))
    raise ValueError(form)


def _f(u, W1, W2, form):
    """The inner model, f(u; W) = GELU(u W1) W2."""
    return _gelu(u @ W1, form) @ W2


def _inner_loss(W1, W2, k, v, loss, form):
    e = _f(k, W1, W2, form) - v
    s = (e * e).sum()
    if loss == "mean":
        return s / v.shape[-1]
    if loss == "sum":
        return s
    raise ValueError(loss)


def _scan_head(Q, K, V, W1_0, W2_0, eta, b, loss, form):
    """One head, one direction, primal form: returns Z [T, d] (z_s = f(q_s; W_s))."""
    T = Q.shape[0]
    W1, W2 = W1_0, W2_0
    rows = []
    for start in range(0, T, b):
        stop = min(start + b, T)
        # every token of the mini-batch takes its gradient at the mini-batch's start state
        grads = [torch.autograd.grad(_inner_loss(W1, W2, K[s], V[s], loss, form), (W1, W2), create_graph=True)
                 for s in range(start, stop)]
        S1, S2 = W1, W2
        for (g1, g2), s in zip(grads, range(start, stop)):
            S1 = S1 - eta * g1
            S2 = S2 - eta * g2
            rows.append(_f(Q[s], S1, S2, form))  # read out after the token's own step
        W1, W2 = S1, S2
    if not rows:
        return Q.new_zeros((0, Q.shape[1]))
    return torch.stack(rows)


def _direction(X, theta, W1_0, W2_0, alpha, eta, b, reverse, loss, form, heads):
    """One gated direction on torch tensors.  X [B, T, D]; returns Y [B, T, D].
    Heads outside `heads` contribute Z = 0 (their Y is X)."""
    Bn, T, D = X.shape
    H, d, _ = W1_0.shape
    gate = torch.tanh(alpha)
    outs = []
    for s in range(Bn):
        Xin = X[s].flip(0) if reverse else X[s]
        Q, K, V = Xin @ theta[0].T, Xin @ theta[1].T, Xin @ theta[2].T
        cols = []
        for h in range(H):
            sl = slice(h * d, (h + 1) * d)
            if h in heads:
                cols.append(_scan_head(Q[:, sl], K[:, sl], V[:, sl], W1_0[h], W2_0[h], eta, b, loss, form))
            else:
                cols.append(Xin.new_zeros((T, d)))
        Z = torch.cat(cols, dim=1) if cols else Xin.new_zeros((T, 0))
        Y = Xin + gate * Z
        outs.append(Y.flip(0) if reverse else Y)
    return torch.stack(outs)


def _leaves(*arrays):
    return [torch.tensor(np.asarray(a, dtype=np.float64), dtype=torch.float64, requires_grad=True) for a in arrays]


def _heads(H, heads, dY, d):
    if heads is None:
        return set(range(H))
    heads = set(heads)
    # gradients restricted to some heads are exact only if dY is zero on the other heads' channels
    others = [c for h in range(H) if h not in heads for c in range(h * d, (h + 1) * d)]
    if others and np.any(np.asarray(dY)[..., others] != 0):
        raise ValueError("dY must be zero outside the selected heads' channels")
    return heads


def layer_forward(X, theta, W1_0, W2_0, alpha, *, eta, b, reverse=False, loss="mean", gelu_form="erf"):
    """Y of one gated direction (float64 NumPy in and out), from the torch form
    that the gradients below differentiate."""
    X3 = np.asarray(X, dtype=np.float64)
    squeeze = X3.ndim == 2
    if squeeze:
        X3 = X3[None]
    with torch.enable_grad():
        Xt, th, w1, w2, al = _leaves(X3, theta, W1_0, W2_0, alpha)
        Y = _direction(Xt, th, w1, w2, al, eta, b, reverse, loss, gelu_form, set(range(w1.shape[0])))
    Y = Y.detach().numpy()
    return Y[0] if squeeze else Y


def ttt_mlp_backward(X, theta, W1_0, W2_0, alpha, dY, *, eta, b, reverse=False, loss="mean",
                     gelu_form="erf", heads=None):
    """Gradients of L = sum(dY * Y) for one gated direction.  X, dY [B, T, D]
    (or [T, D]); theta [3, D, D]; W1_0 [H, d, m]; W2_0 [H, m, d]; alpha [D].
    heads: optionally only these heads (dY must vanish on the others' channels).
    Returns dict(dX, dtheta, dW1_0, dW2_0, dalpha) as float64 NumPy arrays."""
    X3 = np.asarray(X, dtype=np.float64)
    dY3 = np.asarray(dY, dtype=np.float64)
    squeeze = X3.ndim == 2
    if squeeze:
        X3, dY3 = X3[None], dY3[None]
    H, d, _ = np.shape(W1_0)
    hs = _heads(H, heads, dY3, d)
    with torch.enable_grad():
        Xt, th, w1, w2, al = _leaves(X3, theta, W1_0, W2_0, alpha)
        Y = _direction(Xt, th, w1, w2, al, eta, b, reverse, loss, gelu_form, hs)
        L = (torch.from_numpy(dY3) * Y).sum()
        leaves = (Xt, th, w1, w2, al)
        g = torch.autograd.grad(L, leaves, allow_unused=True) if L.requires_grad else [None] * 5
    g = [np.zeros(t.shape) if gi is None else gi.numpy() for gi, t in zip(g, leaves)]
    dX = g[0][0] if squeeze else g[0]
    return dict(dX=dX, dtheta=g[1], dW1_0=g[2], dW2_0=g[3], dalpha=g[4])


def ttt_mlp_bidir_backward(X, theta, W1_0, W2_0, alpha_f, alpha_b, dY, *, eta, b, loss="mean", gelu_form="erf"):
    """Gradients of L = sum(dY * Y) for the bidirectional layer Y = reverse pass
    (alpha_b) over X' = forward pass (alpha_f) over X, same theta and W_0.
    Returns dict(dX, dtheta, dW1_0, dW2_0, dalpha_f, dalpha_b)."""
    X3 = np.asarray(X, dtype=np.float64)
    dY3 = np.asarray(dY, dtype=np.float64)
    squeeze = X3.ndim == 2
    if squeeze:
        X3, dY3 = X3[None], dY3[None]
    H = np.shape(W1_0)[0]
    hs = set(range(H))
    with torch.enable_grad():
        Xt, th, w1, w2, af, ab = _leaves(X3, theta, W1_0, W2_0, alpha_f, alpha_b)
        Xp = _direction(Xt, th, w1, w2, af, eta, b, False, loss, gelu_form, hs)
        Y = _direction(Xp, th, w1, w2, ab, eta, b, True, loss, gelu_form, hs)
        L = (torch.from_numpy(dY3) * Y).sum()
        leaves = (Xt, th, w1, w2, af, ab)
        g = torch.autograd.grad(L, leaves, allow_unused=True) if L.requires_grad else [None] * 6
    g = [np.zeros(t.shape) if gi is None else gi.numpy() for gi, t in zip(g, leaves)]
    dX = g[0][0] if squeeze else g[0]
    return dict(dX=dX, dtheta=g[1], dW1_0=g[2], dW2_0=g[3], dalpha_f=g[4], dalpha_b=g[5])
