"""GPU parity of the layer's backward (ttt_mlp_backward, ttt_mlp_bidir_backward)
against the fp64 backward oracle (autograd through the primal-form layer) on
the same seeded inputs and upstream gradient.

Tolerance: the backward computes in fp32 throughout (bf16 inputs are exact in
fp32), so every gradient must match to 1e-4 of its own largest magnitude
(max-abs error / max |reference|).  The bidirectional layer with bf16 io rounds
X' to bf16 between the passes, as the forward call does, while the oracle keeps
it in fp64: there the bf16 bar applies, relative L2 <= 2e-2."""
import numpy as np
import pytest

from oracle import ttt_backward_oracle as BO
from test_rnn_layer_amd import workloads as W

from tests._common import device_inputs, f64_inputs, from_device, rel_l2

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL_MAX_TOL = 1e-4
BF16_TOL = 2e-2

_F32 = W.WORKLOADS["tiny_f32"]
CASES = {
    # per-token steps, d = 16, m = 64
    "f32_b1": _F32.replace(T=40, name="f32_b1"),
    # mini-batches with a ragged tail; 75 mini-batches = three checkpoint segments of 32
    "f32_b4_segments": _F32.replace(T=298, H=2, d=8, m=32, b=4, eta=0.2, name="f32_b4_segments"),
    # the sum loss and the tanh GELU
    "f32_sum_tanh": _F32.replace(T=37, H=2, d=8, m=16, b=3, eta=0.02, loss="sum", gelu="tanh",
                                 name="f32_sum_tanh"),
    # the bidir307k head shape (bf16 X and theta), two heads, ragged tail: with algo AUTO the
    # forward pass runs on the fp32 matrix cores (state in registers), with GENERIC on the
    # backward's own steps
    "bf16_d64": W.WORKLOADS["bidir307k"].replace(T=72, H=2, seg_len=0, name="bf16_d64"),
    "bf16_d64_generic": W.WORKLOADS["bidir307k"].replace(T=72, H=2, seg_len=0, name="bf16_d64_generic"),
    # the same shape over six checkpoint segments of 32 mini-batches and a 12-token tail: with algo
    # AUTO the backward scan walks them in one window of segments replayed beforehand
    "bf16_d64_segments": W.WORKLOADS["bidir307k"].replace(T=2700, H=1, seg_len=0, name="bf16_d64_segments"),
    # 18 checkpoint segments (556 mini-batches, a 12-token tail): two windows of replayed segments
    # (16, then 2), so the adjoint crosses from one window's walk to the next through the workspace
    "bf16_d64_windows": W.WORKLOADS["bidir307k"].replace(T=8892, H=1, seg_len=0, name="bf16_d64_windows"),
    # the bigstate307k head shape: a state too large for LDS stays in the workspace
    "bf16_d128_b1": W.WORKLOADS["bigstate307k"].replace(T=24, H=1, seg_len=0, name="bf16_d128_b1"),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from test_rnn_layer_amd import _lib
    _lib.lib()  # the HIP library must load: no fallback
    yield


def _cfg(wl):
    from test_rnn_layer_amd import _lib
    return _lib.make_config(wl.B, wl.T, wl.H, wl.d, wl.m, wl.b, wl.eta, io_dtype=wl.io_dtype, loss=wl.loss,
                            gelu=wl.gelu, algo="generic" if wl.name.endswith("_generic") else "auto")


def _check(name, got, ref, tol=REL_MAX_TOL):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    print(f"  {name}: max-abs {err:.3e} of max |ref| {scale:.3e}", flush=True)
    assert err <= tol * max(scale, 1e-30), (name, err, scale)


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("case", list(CASES))
def test_backward_matches_oracle(case, reverse):
    from test_rnn_layer_amd import _lib
    wl = CASES[case]
    print(f"[backward] case={case} reverse={reverse} B{wl.B} T{wl.T} H{wl.H} d{wl.d} m{wl.m} b{wl.b}", flush=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(wl, inp)
    dy = W.make_dy(wl)
    g = _lib.backward(_cfg(wl), dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"],
                      torch.from_numpy(dy).cuda(), reverse=reverse)
    torch.cuda.synchronize()
    f64 = f64_inputs(wl, inp)
    ref = BO.ttt_mlp_backward(f64["X"], f64["theta"], f64["W1_0"], f64["W2_0"], f64["alpha_f"], dy.astype(np.float64),
                              eta=wl.eta, b=wl.b, reverse=reverse, loss=wl.loss, gelu_form=wl.gelu)
    for k in ["dX", "dtheta", "dW1_0", "dW2_0", "dalpha"]:
        _check(k, from_device(g[k]), ref[k])


@pytest.mark.parametrize("case", ["f32_b1", "f32_b4_segments", "bf16_d64", "bf16_d64_segments"])
def test_bidir_backward_matches_oracle(case):
    from test_rnn_layer_amd import _lib
    wl = CASES[case].replace(alpha_f=0.3, alpha_b=-0.2)  # distinct gates catch a swap
    print(f"[bidir backward] case={case}", flush=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(wl, inp)
    dy = W.make_dy(wl)
    g = _lib.bidir_backward(_cfg(wl), dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"],
                            dev["alpha_b"], torch.from_numpy(dy).cuda())
    torch.cuda.synchronize()
    f64 = f64_inputs(wl, inp)
    ref = BO.ttt_mlp_bidir_backward(f64["X"], f64["theta"], f64["W1_0"], f64["W2_0"], f64["alpha_f"],
                                    f64["alpha_b"], dy.astype(np.float64), eta=wl.eta, b=wl.b, loss=wl.loss,
                                    gelu_form=wl.gelu)
    for k in ["dX", "dtheta", "dW1_0", "dW2_0", "dalpha_f", "dalpha_b"]:
        if wl.io_dtype == "f32":
            _check(k, from_device(g[k]), ref[k])
        else:
            err = rel_l2(from_device(g[k]), ref[k])
            print(f"  {k}: rel-L2 {err:.3e}", flush=True)
            assert err <= BF16_TOL, (k, err)


def test_backward_properties_bitwise():
    """Determinism; a zero gate passes dY straight through (dX = dY, nothing else
    moves); causality (dY on the first P tokens only leaves dX zero after them),
    all bitwise; and the bidirectional call equals the reversed pass's backward
    followed by the forward pass's backward with dY = the reversed pass's dX (to
    fp32 rounding: here X' comes from the forward call's generic scan, inside the
    bidirectional backward from the backward's own forward steps)."""
    from test_rnn_layer_amd import _lib
    wl = CASES["f32_b4_segments"]
    print("[backward properties]", flush=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(wl, inp)
    cfg = _cfg(wl)
    dy = torch.from_numpy(W.make_dy(wl)).cuda()
    a = _lib.backward(cfg, dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"], dy)
    b = _lib.backward(cfg, dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"], dy)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
    z = _lib.backward(cfg, dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], torch.zeros_like(dev["alpha_f"]), dy)
    torch.cuda.synchronize()
    assert torch.equal(z["dX"], dy)
    for k in ["dtheta", "dW1_0", "dW2_0"]:
        assert not torch.any(z[k]), k
    P = 100
    dyp = torch.from_numpy(W.make_dy(wl, t1=P)).cuda()
    c = _lib.backward(cfg, dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"], dyp)
    torch.cuda.synchronize()
    assert not torch.any(c["dX"][:, P:]) and torch.any(c["dX"][:, :P])
    # the bidirectional chain, bitwise
    fw = _lib.forward(cfg, dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"])
    bd = _lib.bidir_backward(cfg, dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"], dev["alpha_b"], dy)
    r = _lib.backward(cfg, fw["Y"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_b"], dy, reverse=True)
    f = _lib.backward(cfg, dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"], r["dX"])
    torch.cuda.synchronize()
    for got, want in [(bd["dX"], f["dX"]), (bd["dalpha_b"], r["dalpha"]), (bd["dalpha_f"], f["dalpha"]),
                      (bd["dtheta"], f["dtheta"] + r["dtheta"]), (bd["dW1_0"], f["dW1_0"] + r["dW1_0"]),
                      (bd["dW2_0"], f["dW2_0"] + r["dW2_0"])]:
        scale = want.abs().max().item()
        assert (got - want).abs().max().item() <= 1e-5 * scale, scale


def test_backward_f32_matrix_core_forward_properties():
    """The d = 64 backward whose forward pass runs on the fp32 matrix cores (algo AUTO):
    determinism, a zero gate that passes dY straight through with no other gradient, and
    causality (dY on the first P tokens only leaves dX zero after them), all bitwise,
    over six checkpoint segments (two replay windows) and a ragged tail."""
    from test_rnn_layer_amd import _lib
    wl = CASES["bf16_d64_segments"]
    print("[backward properties, fp32 matrix-core forward]", flush=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(wl, inp)
    cfg = _cfg(wl)
    dy = torch.from_numpy(W.make_dy(wl)).cuda()
    a = _lib.backward(cfg, dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"], dy)
    b = _lib.backward(cfg, dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"], dy)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
    z = _lib.backward(cfg, dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], torch.zeros_like(dev["alpha_f"]), dy)
    torch.cuda.synchronize()
    assert torch.equal(z["dX"], dy)
    for k in ["dtheta", "dW1_0", "dW2_0"]:
        assert not torch.any(z[k]), k
    P = 100
    dyp = torch.from_numpy(W.make_dy(wl, t1=P)).cuda()
    c = _lib.backward(cfg, dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"], dyp)
    torch.cuda.synchronize()
    assert not torch.any(c["dX"][:, P:]) and torch.any(c["dX"][:, :P])


@pytest.mark.parametrize("B", [2, 3])
def test_backward_many_chains(B):
    """B H chains at the bidir307k head shape.  Four workgroups per chain fit co-resident up to 64
    chains (a CU each); at B = 2 (96 chains) the walk over the replayed windows runs on two
    workgroups per chain, at B = 3 (144 chains) on one (the adjoint in the workspace).  dY on heads
    0 and H-1 of every sequence (three checkpoint segments and a ragged tail); the oracle on those
    heads gives every gradient."""
    from test_rnn_layer_amd import _lib
    wl = W.WORKLOADS["bidir307k"].replace(B=B, T=1100, seg_len=0, name="many_chains")
    heads = [0, wl.H - 1]
    print(f"[backward many chains] B{wl.B} H{wl.H} T{wl.T}, dY on heads {heads}", flush=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(wl, inp)
    dy = W.make_dy(wl, heads=heads)
    g = _lib.backward(_cfg(wl), dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"],
                      torch.from_numpy(dy).cuda())
    torch.cuda.synchronize()
    f64 = f64_inputs(wl, inp)
    ref = BO.ttt_mlp_backward(f64["X"], f64["theta"], f64["W1_0"], f64["W2_0"], f64["alpha_f"], dy.astype(np.float64),
                              eta=wl.eta, b=wl.b, loss=wl.loss, gelu_form=wl.gelu, heads=heads)
    for k in ["dX", "dtheta", "dW1_0", "dW2_0", "dalpha"]:
        _check(k, from_device(g[k]), ref[k])


def test_backward_no_tokens():
    from test_rnn_layer_amd import _lib
    wl = CASES["f32_b1"].replace(T=0)
    inp = W.make_inputs(wl)
    dev = device_inputs(wl, inp)
    g = _lib.backward(_cfg(wl), dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"],
                      torch.zeros_like(dev["X"], dtype=torch.float32))
    torch.cuda.synchronize()
    for k in ["dtheta", "dW1_0", "dW2_0", "dalpha"]:
        assert not torch.any(g[k]), k


def test_backward_full_size_prefix():
    """bidir307k's shape (307,200 tokens, 48 heads, bf16 X and theta), the benchmark's
    launch configuration: the forward direction's backward with dY on the first 64
    tokens of heads 0 and 47 against the oracle on that prefix (a causal pass's
    gradients do not depend on later tokens, nor on heads without gradient), and dX
    exactly zero after the prefix."""
    from test_rnn_layer_amd import _lib
    wl = W.WORKLOADS["bidir307k"]
    P, heads = 64, [0, W.WORKLOADS["bidir307k"].H - 1]
    print(f"[backward full size] {wl.name} T={wl.T}, dY on the first {P} tokens of heads {heads}", flush=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(wl, inp)
    dy = W.make_dy(wl, t1=P, heads=heads)
    g = _lib.backward(_cfg(wl), dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"],
                      torch.from_numpy(dy).cuda())
    torch.cuda.synchronize()
    assert not torch.any(g["dX"][:, P:])
    got = {k: from_device(v[:, :P] if k == "dX" else v) for k, v in g.items()}
    del g, dev
    torch.cuda.empty_cache()
    sub = wl.replace(T=P)
    f64 = f64_inputs(sub, dict(inp, X=inp["X"][:, :P]))
    ref = BO.ttt_mlp_backward(f64["X"], f64["theta"], f64["W1_0"], f64["W2_0"], f64["alpha_f"],
                              dy[:, :P].astype(np.float64), eta=wl.eta, b=wl.b, loss=wl.loss, gelu_form=wl.gelu,
                              heads=heads)
    for k in ["dX", "dtheta", "dW1_0", "dW2_0", "dalpha"]:
        _check(k, got[k], ref[k])


def test_backward_full_size_reversed_suffix():
    """The reversed direction at bidir307k's shape: dY on the last 64 tokens of heads 0
    and 47.  In scan order those are the first 64 positions, so the backward walks every
    checkpoint segment of the sequence (with a zero adjoint) before it reaches them; the
    reversed pass over the last 64 tokens alone starts from W_0 at token T-1 and cuts the
    same mini-batches, so the oracle on that suffix gives every gradient, and dX is exactly
    zero before it."""
    from test_rnn_layer_amd import _lib
    wl = W.WORKLOADS["bidir307k"]
    P, heads = 64, [0, wl.H - 1]
    T = wl.T
    print(f"[backward full size, reversed] {wl.name} T={T}, dY on the last {P} tokens of heads {heads}", flush=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(wl, inp)
    dy = np.zeros((wl.B, T, wl.D), dtype=np.float32)
    dy[:, T - P:] = W.make_dy(wl.replace(T=P), heads=heads)
    g = _lib.backward(_cfg(wl), dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"],
                      torch.from_numpy(dy).cuda(), reverse=True)
    torch.cuda.synchronize()
    assert not torch.any(g["dX"][:, :T - P])
    got = {k: from_device(v[:, T - P:] if k == "dX" else v) for k, v in g.items()}
    del g, dev
    torch.cuda.empty_cache()
    sub = wl.replace(T=P)
    f64 = f64_inputs(sub, dict(inp, X=inp["X"][:, T - P:]))
    ref = BO.ttt_mlp_backward(f64["X"], f64["theta"], f64["W1_0"], f64["W2_0"], f64["alpha_f"],
                              dy[:, T - P:].astype(np.float64), eta=wl.eta, b=wl.b, reverse=True, loss=wl.loss,
                              gelu_form=wl.gelu, heads=heads)
    for k in ["dX", "dtheta", "dW1_0", "dW2_0", "dalpha"]:
        _check(k, got[k], ref[k])
