"""Plain fp64 CPU oracle of the TTT-Linear layer (test infrastructure only).

Like ttt_oracle, this module is the checker, not the product: only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it.  It shares
no code with the HIP library.

What it computes: "One-Minute Video Generation with Test-Time Training",
paper-notes page.  Its ablation table lists TTT-Linear beside TTT-MLP: the same
layer with a linear hidden state.  Everything else follows the page's "key
designs" ("TTT-MLP layer", "gate + bidirectional") as in ttt_oracle:

* the inner model is f(u; W) = u W, W a d x d matrix per head (tokens are
  rows, no bias);
* every token takes a gradient step on l(W; x_t) = ||k_t W - v_t||^2 (mean
  reading: divided by d; "sum": the literal square), k_t = theta_K x_t,
  v_t = theta_V x_t; its gradient is k_t^T g_t with g_t = c (k_t W - v_t),
  c = 2/d (mean) or 2 (sum);
* z_t = q_t W_t reads out with the state after token t's own step;
* y = x + tanh(alpha) z per channel; the bidirectional layer runs forward,
  then reversed over the forward output with its own gate and the same
  theta and W_0.

The readings of ttt_oracle's header hold unchanged (mean loss by default,
theta [out, in], head h owns channels [h d, (h+1) d), mini-batches of b
tokens take all their gradients at the state they start from, a final short
mini-batch, sequential bidirectional composition).  The scan is in primal
form: every token's state is materialised, in float64.
"""
from __future__ import annotations

from concurrent.futures import ProcessPoolExecutor

import numpy as np

from oracle.ttt_oracle import _loss_scale, _one_blas_thread, default_workers, project

__all__ = ["linear_loss", "linear_grad", "scan_head_linear", "ttt_linear_forward", "ttt_linear_bidir",
           "default_workers"]


def linear_loss(W, k, v, loss: str = "mean") -> float:
    """l(W; x) = ||k W - v||^2, averaged over d ("mean") or summed ("sum")."""
    e = np.asarray(k) @ W - v
    s = float(e @ e)
    return s / len(v) if loss == "mean" else s


def linear_grad(W, K, V, loss: str = "mean"):
    """Gradient of l(W; x_s) w.r.t. W for each row s of K, V: k_s^T g_s with
    g_s = c (k_s W - v_s).  Returns [n, d, d]."""
    K = np.atleast_2d(K)
    V = np.atleast_2d(V)
    c = _loss_scale(W.shape[1], loss)
    G = c * (K @ W - V)
    return np.einsum("si,sj->sij", K, G)


def scan_head_linear(Q, K, V, W_0, eta: float, b: int, loss: str = "mean"):
    """One head, one direction.  Q, K, V [T, d]; W_0 [d, d].

    Returns (Z [T, d], W_T) with Z[t] = q_t W_t.
    """
    T, d = Q.shape
    W = np.array(W_0, dtype=np.float64)
    Z = np.zeros((T, d))
    for start in range(0, T, b):
        stop = min(start + b, T)
        dW = linear_grad(W, K[start:stop], V[start:stop], loss)  # all at the mini-batch's start state
        S = W.copy()
        for i, s in enumerate(range(start, stop)):
            S -= eta * dW[i]  # W_s: the start state minus the steps of tokens <= s
            Z[s] = Q[s] @ S
        W = S
    return Z, W


def _scan_job(args):
    return scan_head_linear(*args)


def _run_heads(jobs, workers: int):
    if workers <= 1 or len(jobs) <= 1:
        return [scan_head_linear(*j) for j in jobs]
    with ProcessPoolExecutor(max_workers=min(workers, len(jobs)), initializer=_one_blas_thread) as ex:
        return list(ex.map(_scan_job, jobs))


def ttt_linear_forward(X, theta, W_0, alpha, *, eta: float, b: int, reverse: bool = False, loss: str = "mean",
                       workers: int = 1, heads=None):
    """One gated direction.  X [B, T, D] (or [T, D]); theta [3, D, D]; W_0 [H, d, d];
    alpha [D].  Returns dict(Y, Z, W_T [B, nh, d, d]); Y = X + tanh(alpha) * Z."""
    X = np.asarray(X, dtype=np.float64)
    squeeze = X.ndim == 2
    if squeeze:
        X = X[None]
    Bn, T, D = X.shape
    H, d, d2 = W_0.shape
    assert d == d2 and H * d == D
    heads = list(range(H)) if heads is None else list(heads)
    nh = len(heads)
    cols = np.concatenate([np.arange(h * d, (h + 1) * d) for h in heads]) if heads else np.zeros(0, int)
    theta = np.asarray(theta, dtype=np.float64)
    W_0 = np.asarray(W_0, dtype=np.float64)
    gate = np.tanh(np.asarray(alpha, dtype=np.float64))[cols]
    Y = np.empty((Bn, T, nh * d))
    Z = np.empty((Bn, T, nh * d))
    W_T = np.empty((Bn, nh, d, d))
    for s in range(Bn):
        Xin = X[s, ::-1] if reverse else X[s]
        Qh, Kh, Vh = project(np.ascontiguousarray(Xin), theta, H, heads)
        res = _run_heads([(Qh[i], Kh[i], Vh[i], W_0[h], eta, b, loss) for i, h in enumerate(heads)], workers)
        Zs = np.empty((T, nh * d))
        for i, (Zh, w) in enumerate(res):
            Zs[:, i * d:(i + 1) * d] = Zh
            W_T[s, i] = w
        Ys = Xin[:, cols] + gate * Zs
        if reverse:
            Zs, Ys = Zs[::-1], Ys[::-1]
        Z[s], Y[s] = Zs, Ys
    if squeeze:
        Y, Z = Y[0], Z[0]
    return dict(Y=Y, Z=Z, W_T=W_T)


def ttt_linear_bidir(X, theta, W_0, alpha_f, alpha_b, *, eta: float, b: int, loss: str = "mean", workers: int = 1):
    """X' = forward pass with alpha_f, then the reversed pass on X' with alpha_b
    (same theta, same W_0).  Returns dict(Y, Xp, Z_f, Z_b, W_Tf, W_Tb)."""
    kw = dict(eta=eta, b=b, loss=loss, workers=workers)
    f = ttt_linear_forward(X, theta, W_0, alpha_f, reverse=False, **kw)
    r = ttt_linear_forward(f["Y"], theta, W_0, alpha_b, reverse=True, **kw)
    return dict(Y=r["Y"], Xp=f["Y"], Z_f=f["Z"], Z_b=r["Z"], W_Tf=f["W_T"], W_Tb=r["W_T"])
