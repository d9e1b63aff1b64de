"""Plain fp64 CPU oracle of the hybrid block's segment-local attention (test
infrastructure only).

Like ttt_oracle, this module is the checker, not the product: only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it.  It shares
no code with the HIP library.

What it computes: "One-Minute Video Generation with Test-Time Training",
paper-notes page, framework section: every block runs self-attention locally,
within each 3-second segment of the video (about 14,400 tokens), and the
gated bidirectional TTT layer globally over the whole sequence.  The pages
give no more detail of the attention; the plainest reading taken here:

* multi-head softmax attention, H heads of width d (head h owns channels
  [h d, (h+1) d) as in the TTT layer), scores q k^T / sqrt(d), every query
  attending to every key of its own segment (no causal mask: the segment is
  a clip of a video, not a sequence to continue); segments are [s L, (s+1) L)
  with a short last one;
* projections Q|K|V = X theta_A^T (theta_A [3 D, D], [out, in]) and the output
  projection O theta_O^T (theta_O [D, D]), no biases and no norms, a residual
  connection: U = X + attention(X) theta_O^T;
* the block: Y = the bidirectional gated TTT-MLP layer over U (ttt_oracle's
  ttt_bidir).

Everything is float64.
"""
from __future__ import annotations

import numpy as np

from oracle import ttt_oracle as O

__all__ = ["segment_attention", "attention_sublayer", "hybrid_block"]


def segment_attention(Q, K, V, seg_len: int, H: int):
    """Q, K, V [T, D] (or [B, T, D]); returns O of the same shape: for each
    segment [s L, (s+1) L) and head, softmax(Q K^T / sqrt(d)) V over the
    segment's keys."""
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    squeeze = Q.ndim == 2
    if squeeze:
        Q, K, V = Q[None], K[None], V[None]
    Bn, T, D = Q.shape
    d = D // H
    out = np.zeros_like(Q)
    scale = 1.0 / np.sqrt(d)
    for b in range(Bn):
        for s0 in range(0, T, seg_len):
            s1 = min(s0 + seg_len, T)
            for h in range(H):
                c = slice(h * d, (h + 1) * d)
                S = Q[b, s0:s1, c] @ K[b, s0:s1, c].T * scale
                S -= S.max(axis=1, keepdims=True)  # exact: softmax is shift-invariant
                P = np.exp(S)
                P /= P.sum(axis=1, keepdims=True)
                out[b, s0:s1, c] = P @ V[b, s0:s1, c]
    return out[0] if squeeze else out


def attention_sublayer(X, theta_A, theta_O, seg_len: int, H: int):
    """U = X + attention(X theta_A^T) theta_O^T.  X [B, T, D]; theta_A [3, D, D]
    (Q, K, V projections, each [out, in]); theta_O [D, D] ([out, in]).
    Returns dict(U, QKV [B, T, 3 D], O [B, T, D])."""
    X = np.asarray(X, dtype=np.float64)
    thA = np.asarray(theta_A, dtype=np.float64)
    thO = np.asarray(theta_O, dtype=np.float64)
    Q, K, V = X @ thA[0].T, X @ thA[1].T, X @ thA[2].T
    Oa = segment_attention(Q, K, V, seg_len, H)
    return dict(U=X + Oa @ thO.T, QKV=np.concatenate([Q, K, V], axis=-1), O=Oa)


def hybrid_block(X, theta_A, theta_O, seg_len: int, theta, W1_0, W2_0, alpha_f, alpha_b, *, eta: float, b: int,
                 loss: str = "mean", gelu_form: str = "erf", workers: int = 1):
    """The block: U = X + segment attention, then the bidirectional gated
    TTT-MLP layer over U.  Returns dict(Y, U) (and the TTT layer's other outputs)."""
    H = np.shape(W1_0)[0]
    a = attention_sublayer(X, theta_A, theta_O, seg_len, H)
    r = O.ttt_bidir(a["U"], theta, W1_0, W2_0, alpha_f, alpha_b, eta=eta, b=b, loss=loss, gelu_form=gelu_form,
                    workers=workers)
    return dict(r, U=a["U"], O=a["O"])
