"""Plain fp64 CPU oracle of the TTT-MLP layer (test infrastructure only).

This module is the checker, not the product: only the tests, the smoke check
and the benchmark's CPU-baseline leg may import it.  It shares no code with
the HIP library and imports nothing from it.

What it computes follows "One-Minute Video Generation with Test-Time
Training", paper-notes page, section "key designs":

* "TTT-MLP layer": the hidden state is a two-layer MLP with hidden width 4x
  the input width and a GELU, f(u; W) = GELU(u W1) W2 (tokens are rows).  For
  every token it takes a gradient step on the self-supervised loss
  l(W; x_t) = || f(theta_K x_t; W) - theta_V x_t ||^2 and emits
  z_t = f(theta_Q x_t; W_t) with the state *after* that token's step.
  theta_K, theta_V, theta_Q are learned like attention's K, V, Q.
* "gate + bidirectional": gate(TTT, X; alpha) = tanh(alpha) (x) TTT(X) + X
  with a learned gate vector alpha; the layer runs forward, then reversed,
  the two directions sharing the TTT parameters and having their own gate.

Readings taken where the pages are silent (each is a switch or a documented
choice; none is invented arithmetic):

* loss reduction: "mean" uses (1/d)||e||^2, "sum" the literal ||e||^2.  With
  the literal sum the state diverges on every studied configuration, so the
  mean is the default; both stay selectable.
* GELU: the exact erf form by default, the tanh approximation selectable.
* no biases, no normalisation inside f; TTT(X) is the head-major
  concatenation of the per-head outputs z_t.
* theta is stored [out, in] so q_t = theta_Q x_t is the row X @ theta_Q^T;
  head h owns channels [h d, (h+1) d).
* mini-batch size b (b = 1 is the pages' per-token rule): all gradients of a
  mini-batch are taken at the state the mini-batch starts from; token t then
  reads out with that state minus eta times the sum of the gradients of the
  tokens s <= t of its mini-batch; the next mini-batch starts from the state
  of the mini-batch's last token.  A final short mini-batch covers T mod b.
* bidirectional composition is sequential: the reversed pass runs on the
  forward pass's gated output X', restarts from W_0, and cuts its
  mini-batches from the start of the reversed sequence.

The scan is written in its primal form: the state W_t of every token is
materialised.  Everything is float64; inputs are widened exactly and no
intermediate is rounded.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np
from scipy.special import erf

__all__ = [
    "gelu", "gelu_grad", "mlp", "inner_loss", "inner_grad", "project",
    "scan_head", "ttt_forward", "ttt_bidir",
]

_INV_SQRT2 = 1.0 / math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)
_TANH_C = math.sqrt(2.0 / math.pi)
_TANH_K = 0.044715


# ----------------------------------------------------------------------------
# the inner model (page 1, "TTT-MLP layer": two-layer MLP with GELU)
# ----------------------------------------------------------------------------

def gelu(a, form: str = "erf"):
    """GELU(a).  erf form: a * Phi(a) with Phi the standard normal CDF.
    tanh form: 0.5 a (1 + tanh(sqrt(2/pi) (a + 0.044715 a^3)))."""
    a = np.asarray(a, dtype=np.float64)
    if form == "erf":
        return 0.5 * a * (1.0 + erf(a * _INV_SQRT2))
    if form == "tanh":
        return 0.5 * a * (1.0 + np.tanh(_TANH_C * (a + _TANH_K * a ** 3)))
    raise ValueError(form)


def gelu_grad(a, form: str = "erf"):
    """d GELU / d a.  erf form: Phi(a) + a phi(a), phi the normal density."""
    a = np.asarray(a, dtype=np.float64)
    if form == "erf":
        return 0.5 * (1.0 + erf(a * _INV_SQRT2)) + a * _INV_SQRT_2PI * np.exp(-0.5 * a * a)
    if form == "tanh":
        u = _TANH_C * (a + _TANH_K * a ** 3)
        th = np.tanh(u)
        du = _TANH_C * (1.0 + 3.0 * _TANH_K * a * a)
        return 0.5 * (1.0 + th) + 0.5 * a * (1.0 - th * th) * du
    raise ValueError(form)


def mlp(u, W1, W2, form: str = "erf"):
    """f(u; W) = GELU(u W1) W2 for a row (or rows) u."""
    return gelu(np.asarray(u) @ W1, form) @ W2


def _loss_scale(d: int, loss: str) -> float:
    # d/de of (1/d)||e||^2 is (2/d) e; of ||e||^2 it is 2 e
    if loss == "mean":
        return 2.0 / d
    if loss == "sum":
        return 2.0
    raise ValueError(loss)


def inner_loss(W1, W2, k, v, loss: str = "mean", form: str = "erf") -> float:
    """l(W; x) = ||f(k; W) - v||^2, summed ("sum") or averaged over d ("mean")."""
    e = mlp(k, W1, W2, form) - v
    s = float(e @ e)
    return s / len(v) if loss == "mean" else s


def inner_grad(W1, W2, K, V, loss: str = "mean", form: str = "erf"):
    """Gradient of l(W; x_s) w.r.t. W1 and W2 for each row s of K, V.

    Returns (dW1 [n, d, m], dW2 [n, m, d]): per token s,
    a = k W1, h = GELU(a), e = h W2 - v, g2 = c e, g1 = (g2 W2^T) * GELU'(a),
    dW1 = k^T g1, dW2 = h^T g2 (c = 2/d for "mean", 2 for "sum").
    """
    K = np.atleast_2d(K)
    V = np.atleast_2d(V)
    c = _loss_scale(W2.shape[1], loss)
    A = K @ W1
    Hk = gelu(A, form)
    G2 = c * (Hk @ W2 - V)
    G1 = (G2 @ W2.T) * gelu_grad(A, form)
    return np.einsum("si,sj->sij", K, G1), np.einsum("si,sj->sij", Hk, G2)


# ----------------------------------------------------------------------------
# outer-loop projections (page 1, "TTT-MLP layer": theta_K, theta_V, theta_Q)
# ----------------------------------------------------------------------------

def project(X, theta, H: int, heads=None):
    """Q, K, V = X theta_Q^T, X theta_K^T, X theta_V^T, split per head.

    X [T, D], theta [3, D, D] ([out, in]).  Returns three [len(heads), T, d]
    arrays (all H heads by default); head h is channels [h d, (h+1) d) of the
    projection.
    """
    T, D = X.shape
    d = D // H
    heads = list(range(H)) if heads is None else list(heads)
    rows = np.concatenate([np.arange(h * d, (h + 1) * d) for h in heads]) if heads else np.zeros(0, int)
    out = []
    for p in range(3):
        P = X @ theta[p][rows].T
        out.append(np.ascontiguousarray(P.reshape(T, len(heads), d).transpose(1, 0, 2)))
    return out


# ----------------------------------------------------------------------------
# the scan (primal form)
# ----------------------------------------------------------------------------

def scan_head(Q, K, V, W1_0, W2_0, eta: float, b: int, loss: str = "mean", form: str = "erf"):
    """One head, one direction.  Q, K, V [T, d]; W1_0 [d, m]; W2_0 [m, d].

    Returns (Z [T, d], W1_T, W2_T) where Z[t] = f(q_t; W_t).
    """
    T, d = Q.shape
    W1 = np.array(W1_0, dtype=np.float64)
    W2 = np.array(W2_0, dtype=np.float64)
    Z = np.zeros((T, d))
    for start in range(0, T, b):
        stop = min(start + b, T)
        # every gradient of the mini-batch at the state it starts from
        dW1, dW2 = inner_grad(W1, W2, K[start:stop], V[start:stop], loss, form)
        S1, S2 = W1.copy(), W2.copy()
        for i, s in enumerate(range(start, stop)):
            S1 -= eta * dW1[i]  # S = W_s: start state minus the steps of tokens <= s
            S2 -= eta * dW2[i]
            Z[s] = mlp(Q[s], S1, S2, form)
        W1, W2 = S1, S2
    return Z, W1, W2


def _scan_job(args):
    return scan_head(*args)


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass


def _run_heads(jobs, workers: int):
    if workers <= 1 or len(jobs) <= 1:
        return [scan_head(*j) for j in jobs]
    with ProcessPoolExecutor(max_workers=min(workers, len(jobs)), initializer=_one_blas_thread) as ex:
        return list(ex.map(_scan_job, jobs))


def ttt_forward(X, theta, W1_0, W2_0, alpha, *, eta: float, b: int, reverse: bool = False,
                loss: str = "mean", gelu_form: str = "erf", workers: int = 1, heads=None):
    """One gated direction of the layer.

    X [B, T, D] float64 (or [T, D]); theta [3, D, D]; W1_0 [H, d, m];
    W2_0 [H, m, d]; alpha [D].  reverse=True runs over t = T..1.
    heads: optional list of heads to compute (all by default); the outputs
    then hold only those heads' channels, in the order given.
    Returns dict(Y, Z, W1_T [B, nh, d, m], W2_T [B, nh, m, d]);
    Y = X + tanh(alpha) * Z, per channel.
    """
    X = np.asarray(X, dtype=np.float64)
    squeeze = X.ndim == 2
    if squeeze:
        X = X[None]
    Bn, T, D = X.shape
    H, d, m = W1_0.shape
    assert H * d == D
    heads = list(range(H)) if heads is None else list(heads)
    nh = len(heads)
    cols = np.concatenate([np.arange(h * d, (h + 1) * d) for h in heads]) if heads else np.zeros(0, int)
    theta = np.asarray(theta, dtype=np.float64)
    W1_0 = np.asarray(W1_0, dtype=np.float64)
    W2_0 = np.asarray(W2_0, dtype=np.float64)
    gate = np.tanh(np.asarray(alpha, dtype=np.float64))[cols]
    Y = np.empty((Bn, T, nh * d))
    Z = np.empty((Bn, T, nh * d))
    W1_T = np.empty((Bn, nh, d, m))
    W2_T = np.empty((Bn, nh, m, d))
    for s in range(Bn):
        Xin = X[s, ::-1] if reverse else X[s]
        Qh, Kh, Vh = project(np.ascontiguousarray(Xin), theta, H, heads)
        jobs = [(Qh[i], Kh[i], Vh[i], W1_0[h], W2_0[h], eta, b, loss, gelu_form) for i, h in enumerate(heads)]
        res = _run_heads(jobs, workers)
        Zs = np.empty((T, nh * d))
        for i, (Zh, w1, w2) in enumerate(res):
            Zs[:, i * d:(i + 1) * d] = Zh
            W1_T[s, i], W2_T[s, i] = w1, w2
        Ys = Xin[:, cols] + gate * Zs
        if reverse:
            Zs, Ys = Zs[::-1], Ys[::-1]
        Z[s], Y[s] = Zs, Ys
    if squeeze:
        Y, Z = Y[0], Z[0]
    return dict(Y=Y, Z=Z, W1_T=W1_T, W2_T=W2_T)


def ttt_bidir(X, theta, W1_0, W2_0, alpha_f, alpha_b, *, eta: float, b: int,
              loss: str = "mean", gelu_form: str = "erf", workers: int = 1):
    """The bidirectional gated layer: X' = forward pass with alpha_f, then the
    reversed pass on X' with alpha_b (same theta, same W_0).

    Returns dict(Y, Xp, Z_f, Z_b, W1_Tf, W2_Tf, W1_Tb, W2_Tb).
    """
    kw = dict(eta=eta, b=b, loss=loss, gelu_form=gelu_form, workers=workers)
    f = ttt_forward(X, theta, W1_0, W2_0, alpha_f, reverse=False, **kw)
    r = ttt_forward(f["Y"], theta, W1_0, W2_0, alpha_b, reverse=True, **kw)
    return dict(Y=r["Y"], Xp=f["Y"], Z_f=f["Z"], Z_b=r["Z"], W1_Tf=f["W1_T"], W2_Tf=f["W2_T"],
                W1_Tb=r["W1_T"], W2_Tb=r["W2_T"])


def default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))
