"""Pins of the segment-attention oracle (oracle/attention_oracle.py) to things
other than itself: closed forms (equal keys give the mean of the values, a
one-token segment gives its value, a dominant key selects its value), the
softmax's invariances (a shift of one query's scores, a common permutation of
keys and values), segment independence, torch's scaled-dot-product attention
as a second implementation, and the block's reduction to the TTT layer when
the attention's output projection is zero.  CPU only."""
import numpy as np
import pytest

from oracle import attention_oracle as AO
from oracle import ttt_oracle as O


def _qkv(seed, T=10, H=2, d=4, B=1):
    rng = np.random.default_rng(seed)
    D = H * d
    return [rng.normal(size=(B, T, D)) for _ in range(3)]


def test_equal_keys_give_the_mean_value():
    Q, K, V = _qkv(1, T=9)
    K[:] = K[:, :1]  # every key equal: uniform weights within each segment
    out = AO.segment_attention(Q, K, V, seg_len=4, H=2)
    for s0 in range(0, 9, 4):
        s1 = min(s0 + 4, 9)
        np.testing.assert_allclose(out[:, s0:s1], np.broadcast_to(V[:, s0:s1].mean(axis=1, keepdims=True),
                                                                   out[:, s0:s1].shape), rtol=1e-13, atol=1e-14)


def test_one_token_segments_return_their_value():
    Q, K, V = _qkv(2, T=7)
    np.testing.assert_allclose(AO.segment_attention(Q, K, V, seg_len=1, H=2), V, rtol=0, atol=1e-15)


def test_dominant_key_selects_its_value():
    Q, K, V = _qkv(3, T=6, H=1, d=4)
    K[0, 2] = Q[0, 0] * 200.0  # query 0's score on key 2 exceeds the others by thousands
    out = AO.segment_attention(Q, K, V, seg_len=6, H=1)
    np.testing.assert_allclose(out[0, 0], V[0, 2], rtol=0, atol=1e-12)


def test_permutation_of_keys_and_values_and_shift_invariance():
    Q, K, V = _qkv(4, T=8)
    perm = np.random.default_rng(5).permutation(8)
    a = AO.segment_attention(Q, K, V, seg_len=8, H=2)
    b = AO.segment_attention(Q, K[:, perm], V[:, perm], seg_len=8, H=2)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    # a key component along nothing but one query changes no weight if added to every key:
    # adding the same vector c to every key shifts each query's scores by q.c
    c = np.random.default_rng(6).normal(size=(1, 1, K.shape[-1]))
    np.testing.assert_allclose(AO.segment_attention(Q, K + c, V, seg_len=8, H=2), a, rtol=1e-11, atol=1e-12)


def test_segments_are_independent():
    Q, K, V = _qkv(7, T=12)
    a = AO.segment_attention(Q, K, V, seg_len=5, H=2)
    K2, V2 = K.copy(), V.copy()
    K2[:, 5:10] += 3.0
    V2[:, 5:10] -= 1.0
    b = AO.segment_attention(Q, K2, V2, seg_len=5, H=2)
    np.testing.assert_array_equal(a[:, :5], b[:, :5])
    np.testing.assert_array_equal(a[:, 10:], b[:, 10:])
    assert not np.allclose(a[:, 5:10], b[:, 5:10])


def test_matches_torch_sdpa():
    torch = pytest.importorskip("torch")
    Q, K, V = _qkv(8, T=11, H=3, d=5, B=2)
    L = 4
    out = AO.segment_attention(Q, K, V, seg_len=L, H=3)
    for s0 in range(0, 11, L):
        s1 = min(s0 + L, 11)
        t = [torch.from_numpy(a[:, s0:s1]).reshape(2, s1 - s0, 3, 5).transpose(1, 2) for a in (Q, K, V)]
        ref = torch.nn.functional.scaled_dot_product_attention(*t).transpose(1, 2).reshape(2, s1 - s0, 15).numpy()
        np.testing.assert_allclose(out[:, s0:s1], ref, rtol=1e-12, atol=1e-12)


def test_block_with_zero_output_projection_is_the_ttt_layer():
    rng = np.random.default_rng(9)
    H, d, m, T = 2, 4, 8, 10
    D = H * d
    X = rng.normal(size=(1, T, D))
    thA = rng.normal(size=(3, D, D)) / np.sqrt(D)
    th = rng.normal(size=(3, D, D)) / np.sqrt(D)
    W1 = rng.normal(size=(H, d, m)) / np.sqrt(d)
    W2 = rng.normal(size=(H, m, d)) / np.sqrt(m)
    af, ab = np.full(D, 0.3), np.full(D, -0.2)
    kw = dict(eta=0.1, b=3)
    blk = AO.hybrid_block(X, thA, np.zeros((D, D)), 4, th, W1, W2, af, ab, **kw)
    ref = O.ttt_bidir(X, th, W1, W2, af, ab, **kw)
    np.testing.assert_array_equal(blk["U"], X)
    np.testing.assert_array_equal(blk["Y"], ref["Y"])
    # and with an output projection, U = X + O theta_O^T
    thO = rng.normal(size=(D, D)) / np.sqrt(D)
    a = AO.attention_sublayer(X, thA, thO, 4, H)
    np.testing.assert_allclose(a["U"] - X, a["O"] @ thO.T, rtol=1e-13, atol=1e-13)
