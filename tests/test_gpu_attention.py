"""GPU parity of the segment-local attention and the hybrid block (segment
attention feeding the bidirectional TTT layer) against the fp64 oracle on the
same inputs.

Tolerance: bf16 io, relative L2 <= 2e-2 (the project's bar for bf16-input
paths).  The attention rounds the probabilities to bf16 as matrix operands
(relative error 2^-9 each) and its output to bf16; measured errors are printed."""
import numpy as np
import pytest

from oracle import attention_oracle as AO
from test_rnn_layer_amd import workloads as W

from tests._common import device_inputs, f64_inputs, from_device, rel_l2, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from test_rnn_layer_amd import _lib
    _lib.lib()  # the HIP library must load: no fallback
    yield


def _cfg(B, T, H):
    from test_rnn_layer_amd import _lib
    return _lib.make_config(B, T, H, 64, 256, 16, 0.1 / 16, io_dtype="bf16")


def _qkv(B, T, H, seed):
    """Seeded N(0, 1) Q | K | V on the device (bf16) and its exact fp64 copy."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    qkv = torch.randn((B, T, 3 * H * 64), generator=g, device="cuda").to(torch.bfloat16)
    return qkv, from_device(qkv)


def _oracle(q64, H, L):
    D = H * 64
    return AO.segment_attention(q64[..., :D], q64[..., D:2 * D], q64[..., 2 * D:], L, H)


CASES = [  # B, T, H, L
    (1, 300, 2, 100),   # three segments of 100: one query tile each, ragged key blocks
    (2, 257, 1, 200),   # a 200-token segment (two query tiles) and a 57-token one, two sequences
    (1, 1000, 1, 1000),  # one segment of 8 query tiles and 16 key blocks, the last ragged
    (1, 37, 2, 5),      # many tiny segments
    (1, 90, 3, 4096),   # a segment longer than the sequence
]


@pytest.mark.parametrize("B,T,H,L", CASES)
def test_segment_attention_matches_oracle(B, T, H, L):
    from test_rnn_layer_amd import _lib
    print(f"[attention] B{B} T{T} H{H} L{L}", flush=True)
    qkv, q64 = _qkv(B, T, H, seed=B * 1000 + T + L)
    O = _lib.segment_attention(_cfg(B, T, H), L, qkv)
    torch.cuda.synchronize()
    err = rel_l2(from_device(O), _oracle(q64, H, L))
    print(f"  O: rel-L2 {err:.3e}", flush=True)
    assert err <= BF16_TOL


def test_segment_attention_properties_bitwise():
    """Determinism; a segment's output ignores other segments' keys and values."""
    from test_rnn_layer_amd import _lib
    B, T, H, L = 1, 500, 2, 192
    cfg = _cfg(B, T, H)
    qkv, _ = _qkv(B, T, H, seed=7)
    a = _lib.segment_attention(cfg, L, qkv)
    b = _lib.segment_attention(cfg, L, qkv)
    q2 = qkv.clone()
    q2[:, L:2 * L, H * 64:] = -q2[:, L:2 * L, H * 64:]  # K and V of segment 1 only
    c = _lib.segment_attention(cfg, L, q2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(a[:, :L], c[:, :L]) and torch.equal(a[:, 2 * L:], c[:, 2 * L:])
    assert not torch.equal(a[:, L:2 * L], c[:, L:2 * L])


def test_hybrid_block_matches_oracle():
    from test_rnn_layer_amd import _lib
    wl = W.WORKLOADS["hybrid307k"].replace(T=160, H=2, seg_len=0, attn_seg=48, name="hybrid_small")
    print(f"[hybrid block] T{wl.T} H{wl.H} segments of {wl.attn_seg}", flush=True)
    inp = W.make_inputs(wl)
    thA, thO = W.make_attention_weights(wl)
    dev = device_inputs(wl, inp)
    cfg = _cfg(wl.B, wl.T, wl.H)
    Y = _lib.hybrid_block(cfg, wl.attn_seg, dev["X"], to_device(thA, "bf16"), to_device(thO, "bf16"), dev["theta"],
                          dev["W1_0"], dev["W2_0"], dev["alpha_f"], dev["alpha_b"])
    torch.cuda.synchronize()
    f64 = f64_inputs(wl, inp)
    ref = AO.hybrid_block(f64["X"], W.to_f64(thA, "bf16"), W.to_f64(thO, "bf16"), wl.attn_seg, f64["theta"],
                          f64["W1_0"], f64["W2_0"], f64["alpha_f"], f64["alpha_b"], eta=wl.eta, b=wl.b)
    err = rel_l2(from_device(Y) - f64["X"], ref["Y"] - f64["X"])  # relative to the block's change of X
    print(f"  Y - X: rel-L2 {err:.3e}", flush=True)
    assert err <= BF16_TOL


def test_segment_attention_full_size():
    """hybrid307k's attention shape (307,200 tokens, 48 heads, segments of 14,400, the
    last one 4,800): the first and the last segment of heads 0 and 47 against the
    oracle."""
    from test_rnn_layer_amd import _lib
    wl = W.WORKLOADS["hybrid307k"]
    B, T, H, L = wl.B, wl.T, wl.H, wl.attn_seg
    print(f"[attention full size] T{T} H{H} L{L}", flush=True)
    qkv, _ = _qkv(B, T, H, seed=11)
    O = _lib.segment_attention(_cfg(B, T, H), L, qkv)
    torch.cuda.synchronize()
    D = H * 64
    for s0, s1 in [(0, L), (T - T % L, T)]:
        for h in (0, H - 1):
            cols = [p * D + h * 64 + j for p in range(3) for j in range(64)]
            q64 = from_device(qkv[:, s0:s1][..., cols])
            ref = _oracle(q64, 1, L)
            err = rel_l2(from_device(O[:, s0:s1, h * 64:(h + 1) * 64]), ref)
            print(f"  segment [{s0}, {s1}) head {h}: rel-L2 {err:.3e}", flush=True)
            assert err <= BF16_TOL
