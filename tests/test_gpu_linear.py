"""GPU parity of the TTT-Linear layer (linear inner model, d x d state): the HIP
library through the C ABI against the fp64 linear oracle on the same seeded inputs.

Tolerances as for the MLP layer: fp32 io -- max-abs <= 1e-4 on Y, Z and the
final state; bf16 io -- relative L2 <= 2e-2.
"""
import numpy as np
import pytest

from oracle import ttt_linear_oracle as LO
from test_rnn_layer_amd import workloads as W

from tests._common import device_inputs, f64_inputs, from_device, max_abs, rel_l2, workers

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-4
ALGOS = ["generic", "mfma"]

_BASE = W.WORKLOADS["linear307k"]
CASES = {
    # several mini-batch tiles plus a ragged tail where b > 1
    "lin_h3_b16_ragged": _BASE.replace(T=200, H=3, seg_len=0, name="lin_h3_b16_ragged"),
    # more than one chunked launch per direction on the MFMA path (512 + 768 + 720 tokens)
    "lin_h2_b16_chunks": _BASE.replace(T=2000, H=2, seg_len=0, name="lin_h2_b16_chunks"),
    "lin_seg_shift": _BASE.replace(T=512, H=2, seg_len=160, name="lin_seg_shift"),
    "lin_two_sequences": _BASE.replace(B=2, T=64, H=2, seg_len=0, name="lin_two_sequences"),
    "lin_one_token": _BASE.replace(T=1, H=2, seg_len=0, name="lin_one_token"),
    "lin_shorter_than_b": _BASE.replace(T=9, H=2, seg_len=0, name="lin_shorter_than_b"),
    "lin_sum_loss": _BASE.replace(T=77, H=2, seg_len=0, loss="sum", eta=0.1 / 16 / 64, name="lin_sum_loss"),
    "lin_f32_d16_b4": W.WORKLOADS["tiny_f32"].replace(T=103, d=16, m=16, b=4, model="linear", name="lin_f32_d16_b4"),
    "lin_f32_d32_b1": W.WORKLOADS["tiny_f32"].replace(T=50, H=2, d=32, m=32, b=1, eta=0.05, model="linear",
                                                      name="lin_f32_d32_b1"),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from test_rnn_layer_amd import _lib
    _lib.lib()  # the HIP library must load: no fallback
    yield


def _cfg(wl, algo="auto", T=None):
    from test_rnn_layer_amd import _lib
    return _lib.make_config(wl.B, wl.T if T is None else T, wl.H, wl.d, wl.m, wl.b, wl.eta, io_dtype=wl.io_dtype,
                            loss=wl.loss, algo=algo, model="linear")


def _skip_unsupported(wl, algo):
    from test_rnn_layer_amd import _lib
    try:
        _lib.select_algo(_cfg(wl, algo))
    except _lib.TTTError as e:
        if e.status == _lib.TTT_ERR_UNSUPPORTED:
            pytest.skip(f"{algo} does not support the linear model at d={wl.d} b={wl.b} io={wl.io_dtype}")
        raise


def _forward(wl, dev, algo, reverse=False, alpha="alpha_f", X=None, W0=None, T=None):
    from test_rnn_layer_amd import _lib
    r = _lib.forward(_cfg(wl, algo, T), dev["X"] if X is None else X, dev["theta"], dev["W1_0"] if W0 is None else W0,
                     None, dev[alpha], reverse=reverse, want_z=True, want_state=True)
    torch.cuda.synchronize()
    return r


def _check(name, got, ref, io_dtype):
    if io_dtype == "f32":
        err = max_abs(got, ref)
        print(f"  {name}: max-abs {err:.3e}", flush=True)
        assert err <= F32_TOL, (name, err)
    else:
        err = rel_l2(got, ref)
        print(f"  {name}: rel-L2 {err:.3e}", flush=True)
        assert err <= BF16_TOL, (name, err)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("reverse", [False, True])
def test_linear_forward_matches_oracle(case, reverse, algo):
    wl = CASES[case]
    _skip_unsupported(wl, algo)
    print(f"[linear forward] case={case} reverse={reverse} algo={algo} B{wl.B} T{wl.T} H{wl.H} d{wl.d} b{wl.b}",
          flush=True)
    inp = W.make_inputs(wl)
    got = _forward(wl, device_inputs(wl, inp), algo, reverse=reverse)
    assert got["W2_T"] is None
    f64 = f64_inputs(wl, inp)
    ref = LO.ttt_linear_forward(f64["X"], f64["theta"], f64["W1_0"], f64["alpha_f"], eta=wl.eta, b=wl.b,
                                reverse=reverse, loss=wl.loss, workers=workers())
    _check("Y", from_device(got["Y"]), ref["Y"], wl.io_dtype)
    _check("Z", from_device(got["Z"]), ref["Z"], wl.io_dtype)
    _check("W_T", from_device(got["W1_T"]), ref["W_T"], wl.io_dtype)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("case", ["lin_h3_b16_ragged", "lin_h2_b16_chunks", "lin_f32_d16_b4"])
def test_linear_bidir_matches_oracle(case, algo):
    from test_rnn_layer_amd import _lib
    wl = CASES[case].replace(alpha_f=0.1, alpha_b=0.2)  # distinct gates catch a swap
    _skip_unsupported(wl, algo)
    print(f"[linear bidir] case={case} algo={algo}", flush=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(wl, inp)
    got = _lib.bidir(_cfg(wl, algo), dev["X"], dev["theta"], dev["W1_0"], None, dev["alpha_f"], dev["alpha_b"],
                     want_z=True, want_state=True)
    torch.cuda.synchronize()
    f64 = f64_inputs(wl, inp)
    ref = LO.ttt_linear_bidir(f64["X"], f64["theta"], f64["W1_0"], f64["alpha_f"], f64["alpha_b"], eta=wl.eta,
                              b=wl.b, loss=wl.loss, workers=workers())
    _check("Y", from_device(got["Y"]), ref["Y"], wl.io_dtype)
    _check("Z_f", from_device(got["Z_f"]), ref["Z_f"], wl.io_dtype)
    _check("Z_b", from_device(got["Z_b"]), ref["Z_b"], wl.io_dtype)
    _check("W_Tf", from_device(got["W1_Tf"]), ref["W_Tf"], wl.io_dtype)
    _check("W_Tb", from_device(got["W1_Tb"]), ref["W_Tb"], wl.io_dtype)


@pytest.mark.parametrize("algo", ALGOS)
def test_linear_properties_bitwise(algo):
    """Determinism, reversed pass == forward pass on the flipped sequence, alpha = 0
    leaves X untouched, bidir == forward then reversed forward, and the state
    hand-off (continuing from the state after T1 tokens equals the whole run)."""
    from test_rnn_layer_amd import _lib
    wl = CASES["lin_h2_b16_chunks"]
    _skip_unsupported(wl, algo)
    print(f"[linear properties] algo={algo}", flush=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(wl, inp)
    a = _forward(wl, dev, algo)
    b = _forward(wl, dev, algo)
    assert torch.equal(a["Y"], b["Y"]) and torch.equal(a["Z"], b["Z"]), "not deterministic"
    rv = _forward(wl, dev, algo, reverse=True)
    fl = _forward(wl, dev, algo, X=dev["X"].flip(1).contiguous())
    assert torch.equal(rv["Z"], fl["Z"].flip(1)) and torch.equal(rv["Y"], fl["Y"].flip(1))
    assert torch.equal(rv["W1_T"], fl["W1_T"])
    z = _lib.forward(_cfg(wl, algo), dev["X"], dev["theta"], dev["W1_0"], None, torch.zeros_like(dev["alpha_f"]))
    torch.cuda.synchronize()
    assert torch.equal(z["Y"], dev["X"])
    bd = _lib.bidir(_cfg(wl, algo), dev["X"], dev["theta"], dev["W1_0"], None, dev["alpha_f"], dev["alpha_b"],
                    want_z=True)
    f2 = _forward(wl, dev, algo, reverse=True, alpha="alpha_b", X=a["Y"])
    assert torch.equal(bd["Y"], f2["Y"]) and torch.equal(bd["Z_f"], a["Z"]) and torch.equal(bd["Z_b"], f2["Z"])
    T1 = 1280  # a chunk boundary of the whole run, and a whole number of mini-batches
    first = _forward(wl, dict(dev, X=dev["X"][:, :T1].contiguous()), algo, T=T1)
    rest = _forward(wl, dict(dev, X=dev["X"][:, T1:].contiguous()), algo, T=wl.T - T1,
                    W0=first["W1_T"][0].contiguous())
    assert torch.equal(torch.cat([first["Z"], rest["Z"]], 1), a["Z"])
    assert torch.equal(rest["W1_T"], a["W1_T"])


def test_linear_full_size_bidir():
    """linear307k in the benchmark's launch configuration: the forward pass's first
    2,048 tokens against the oracle (first and last head); the reversed pass
    through bidir == forward then reversed forward on its output, bitwise."""
    from test_rnn_layer_amd import _lib
    wl = W.WORKLOADS["linear307k"]
    prefix = 2048
    print(f"[linear config] {wl.name} full size, prefix {prefix}", flush=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(wl, inp)
    cfg = _cfg(wl)
    r = _lib.bidir(cfg, dev["X"], dev["theta"], dev["W1_0"], None, dev["alpha_f"], dev["alpha_b"], want_z=True)
    f = _lib.forward(cfg, dev["X"], dev["theta"], dev["W1_0"], None, dev["alpha_f"])
    torch.cuda.synchronize()
    assert torch.isfinite(r["Z_b"]).all() and torch.isfinite(r["Y"].float()).all()
    Zf_pre = from_device(r["Z_f"][:, :prefix])
    del r["Z_b"]
    g = _lib.forward(cfg, f["Y"], dev["theta"], dev["W1_0"], None, dev["alpha_b"], reverse=True)
    torch.cuda.synchronize()
    assert torch.equal(g["Y"], r["Y"])
    del dev, r, f, g
    torch.cuda.empty_cache()
    sub = wl.replace(T=prefix)
    f64 = f64_inputs(sub, dict(inp, X=inp["X"][:, :prefix]))
    heads = [0, wl.H - 1]
    ref = LO.ttt_linear_forward(f64["X"], f64["theta"], f64["W1_0"], f64["alpha_f"], eta=wl.eta, b=wl.b,
                                heads=heads, workers=workers())
    cols = np.concatenate([np.arange(h * wl.d, (h + 1) * wl.d) for h in heads])
    _check("Z_f prefix", Zf_pre[:, :, cols], ref["Z"], wl.io_dtype)
