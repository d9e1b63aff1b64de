"""GPU parity: the HIP library against the fp64 oracle on the same seeded inputs.

Tolerances: fp32 io -- max-abs <= 1e-4 on Y, Z and the final state;
bf16 io -- relative L2 <= 2e-2 on Y, Z (each direction) and the final state.
Every call goes through the C ABI (test_rnn_layer_amd._lib).
"""
import numpy as np
import pytest

from oracle import ttt_oracle as O
from test_rnn_layer_amd import workloads as W

from tests._common import device_inputs, f64_inputs, from_device, max_abs, rel_l2, rel_l2_tenths, workers

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-4
ALGOS = ["generic", "mfma", "coop"]


def _skip_unsupported(wl, algo):
    from test_rnn_layer_amd import _lib
    try:
        _lib.select_algo(_cfg(wl, algo))
    except _lib.TTTError as e:
        if e.status == _lib.TTT_ERR_UNSUPPORTED:
            pytest.skip(f"{algo} does not support d={wl.d} m={wl.m} b={wl.b} io={wl.io_dtype}")
        raise


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from test_rnn_layer_amd import _lib
    _lib.lib()  # the HIP library must load: no fallback
    yield


def _cfg(wl, algo="auto", T=None):
    from test_rnn_layer_amd import _lib
    return _lib.make_config(wl.B, wl.T if T is None else T, wl.H, wl.d, wl.m, wl.b, wl.eta,
                            io_dtype=wl.io_dtype, loss=wl.loss, gelu=wl.gelu, algo=algo)


def _gpu_forward(wl, dev, algo, reverse=False, alpha="alpha_f"):
    from test_rnn_layer_amd import _lib
    r = _lib.forward(_cfg(wl, algo), dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev[alpha],
                     reverse=reverse, want_z=True, want_state=True)
    torch.cuda.synchronize()
    return r


def _gpu_bidir(wl, dev, algo):
    from test_rnn_layer_amd import _lib
    r = _lib.bidir(_cfg(wl, algo), dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"],
                   dev["alpha_b"], want_z=True, want_state=True)
    torch.cuda.synchronize()
    return r


def _oracle_forward(wl, f64, reverse=False, alpha="alpha_f"):
    return O.ttt_forward(f64["X"], f64["theta"], f64["W1_0"], f64["W2_0"], f64[alpha], eta=wl.eta, b=wl.b,
                         reverse=reverse, loss=wl.loss, gelu_form=wl.gelu, workers=workers())


def _check(name, got, ref, io_dtype):
    if io_dtype == "f32":
        err = max_abs(got, ref)
        print(f"  {name}: max-abs {err:.3e}", flush=True)
        assert err <= F32_TOL, (name, err)
    else:
        err = rel_l2(got, ref)
        print(f"  {name}: rel-L2 {err:.3e}", flush=True)
        assert err <= BF16_TOL, (name, err)


def _check_forward(wl, got, ref):
    _check("Y", from_device(got["Y"]), ref["Y"], wl.io_dtype)
    _check("Z", from_device(got["Z"]), ref["Z"], wl.io_dtype)
    _check("W1_T", from_device(got["W1_T"]), ref["W1_T"], wl.io_dtype)
    _check("W2_T", from_device(got["W2_T"]), ref["W2_T"], wl.io_dtype)


# ----------------------------------------------------------------------------
# small and medium shapes, element by element
# ----------------------------------------------------------------------------

SMALL = {
    # name: workload (several mini-batch tiles plus a ragged tail where b > 1)
    "tiny_f32": W.WORKLOADS["tiny_f32"],
    "tiny_f32_b4_ragged": W.WORKLOADS["tiny_f32"].replace(T=103, b=4, name="tiny_f32_b4_ragged"),
    "h3_d64_b16_ragged": W.WORKLOADS["seg14k"].replace(T=200, H=3, name="h3_d64_b16_ragged"),
    # several scan launches per direction on the MFMA path (chunks of 512 + 512 + 512 + 467 tokens),
    # so the reversed pass starts launches at positions p0 > 0 and hands its state between them;
    # 2,003 = 125 mini-batches of 16 and a ragged one of 3
    "h2_d64_b16_chunks": W.WORKLOADS["seg14k"].replace(T=2003, H=2, name="h2_d64_b16_chunks"),
    "h2_d128_b1": W.WORKLOADS["bigstate307k"].replace(T=96, H=2, name="h2_d128_b1"),
    "d128_b1_f32_tanh_sum": W.WORKLOADS["bigstate307k"].replace(T=33, H=1, io_dtype="f32", gelu="tanh", loss="sum",
                                                                eta=0.05 / 128, name="d128_b1_f32_tanh_sum"),
    "d128_b1_f32": W.WORKLOADS["bigstate307k"].replace(T=50, H=2, io_dtype="f32", name="d128_b1_f32"),
    "d128_b1_two_sequences": W.WORKLOADS["bigstate307k"].replace(B=2, T=40, H=3, name="d128_b1_two_sequences"),
    "d128_b1_one_token": W.WORKLOADS["bigstate307k"].replace(T=1, H=2, name="d128_b1_one_token"),
    # 5 x 8 heads need 320 cooperating workgroups, more than fit at once: AUTO takes the generic scan
    "d128_b1_many_chains": W.WORKLOADS["bigstate307k"].replace(B=5, T=20, H=8, name="d128_b1_many_chains"),
    "seg_shift_b16": W.WORKLOADS["bidir307k"].replace(T=512, H=2, seg_len=160, name="seg_shift_b16"),
    "sum_loss_tanh": W.WORKLOADS["seg14k"].replace(T=77, H=2, loss="sum", eta=0.1 / 16 / 64, gelu="tanh",
                                                   name="sum_loss_tanh"),
    "tanh_gelu": W.WORKLOADS["seg14k"].replace(T=77, H=2, gelu="tanh", name="tanh_gelu"),
    "sum_loss": W.WORKLOADS["seg14k"].replace(T=77, H=2, loss="sum", eta=0.1 / 16 / 64, name="sum_loss"),
    "two_sequences": W.WORKLOADS["seg14k"].replace(B=2, T=64, H=2, name="two_sequences"),
    "one_token": W.WORKLOADS["seg14k"].replace(T=1, H=2, name="one_token"),
    "shorter_than_b": W.WORKLOADS["seg14k"].replace(T=9, H=2, name="shorter_than_b"),
}


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("case", list(SMALL))
@pytest.mark.parametrize("reverse", [False, True])
def test_forward_matches_oracle(case, reverse, algo):
    wl = SMALL[case]
    _skip_unsupported(wl, algo)
    print(f"[forward] case={case} reverse={reverse} algo={algo} shape=B{wl.B} T{wl.T} H{wl.H} d{wl.d} m{wl.m} b{wl.b}",
          flush=True)
    inp = W.make_inputs(wl)
    got = _gpu_forward(wl, device_inputs(wl, inp), algo, reverse=reverse)
    ref = _oracle_forward(wl, f64_inputs(wl, inp), reverse=reverse)
    _check_forward(wl, got, ref)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("case", ["h3_d64_b16_ragged", "h2_d64_b16_chunks", "h2_d128_b1", "seg_shift_b16",
                                  "tiny_f32_b4_ragged"])
def test_bidir_matches_oracle(case, algo):
    wl = SMALL[case].replace(alpha_f=0.1, alpha_b=0.2)  # distinct gates catch a swap
    _skip_unsupported(wl, algo)
    print(f"[bidir] case={case} algo={algo}", flush=True)
    inp = W.make_inputs(wl)
    got = _gpu_bidir(wl, device_inputs(wl, inp), algo)
    f64 = f64_inputs(wl, inp)
    ref = O.ttt_bidir(f64["X"], f64["theta"], f64["W1_0"], f64["W2_0"], f64["alpha_f"], f64["alpha_b"],
                      eta=wl.eta, b=wl.b, loss=wl.loss, gelu_form=wl.gelu, workers=workers())
    _check("Y", from_device(got["Y"]), ref["Y"], wl.io_dtype)
    _check("Z_f", from_device(got["Z_f"]), ref["Z_f"], wl.io_dtype)
    _check("Z_b", from_device(got["Z_b"]), ref["Z_b"], wl.io_dtype)
    for k in ("W1_Tf", "W2_Tf", "W1_Tb", "W2_Tb"):
        _check(k, from_device(got[k]), ref[k], wl.io_dtype)


# the shape each kernel's property tests run on
PROP_CASE = {"generic": "h3_d64_b16_ragged", "mfma": "h3_d64_b16_ragged", "coop": "h2_d128_b1"}


def test_auto_leaves_the_cooperative_scan_when_it_does_not_fit():
    from test_rnn_layer_amd import _lib
    wl = SMALL["d128_b1_many_chains"]
    assert _lib.select_algo(_cfg(wl)) == "generic"
    assert _lib.select_algo(_cfg(wl.replace(B=1, H=2))) == "coop"
    print("[auto] d=128 b=1: 5 x 8 heads on the generic scan, 1 x 2 on the cooperative one", flush=True)
    inp = W.make_inputs(wl)
    got = _gpu_forward(wl, device_inputs(wl, inp), "auto")
    _check_forward(wl, got, _oracle_forward(wl, f64_inputs(wl, inp)))


@pytest.mark.parametrize("algo", ALGOS)
def test_empty_sequence_returns_initial_state(algo):
    from test_rnn_layer_amd import _lib
    wl = SMALL[PROP_CASE[algo]].replace(T=0)
    print(f"[empty] T=0 algo={algo}", flush=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(wl, inp)
    r = _lib.bidir(_cfg(wl, algo), dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"], dev["alpha_b"],
                   want_z=True, want_state=True)
    torch.cuda.synchronize()
    assert r["Y"].numel() == 0
    np.testing.assert_array_equal(r["W1_Tb"][0].cpu().numpy(), inp["W1_0"])
    np.testing.assert_array_equal(r["W2_Tf"][0].cpu().numpy(), inp["W2_0"])


# ----------------------------------------------------------------------------
# properties that hold at any size (bitwise, on the GPU)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("algo", ALGOS)
def test_properties_bitwise(algo):
    from test_rnn_layer_amd import _lib
    wl = SMALL[PROP_CASE[algo]]
    print(f"[properties] algo={algo}", flush=True)
    inp = W.make_inputs(wl)
    dev = device_inputs(wl, inp)
    cfg = _cfg(wl, algo)
    a = _gpu_forward(wl, dev, algo)
    b = _gpu_forward(wl, dev, algo)
    assert torch.equal(a["Y"], b["Y"]) and torch.equal(a["Z"], b["Z"]), "not deterministic"
    # reversed pass == forward pass on the flipped sequence
    rv = _gpu_forward(wl, dev, algo, reverse=True)
    flipped = dict(dev, X=dev["X"].flip(1).contiguous())
    fl = _gpu_forward(wl, flipped, algo)
    assert torch.equal(rv["Z"], fl["Z"].flip(1)) and torch.equal(rv["Y"], fl["Y"].flip(1))
    assert torch.equal(rv["W1_T"], fl["W1_T"])
    # alpha = 0 leaves X untouched
    z = _lib.forward(cfg, dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], torch.zeros_like(dev["alpha_f"]))
    torch.cuda.synchronize()
    assert torch.equal(z["Y"], dev["X"])
    # bidir == forward (alpha_f) then reversed forward (alpha_b) on its output
    bd = _gpu_bidir(wl, dev, algo)
    f2 = _gpu_forward(wl, dict(dev, X=a["Y"]), algo, reverse=True, alpha="alpha_b")
    assert torch.equal(bd["Y"], f2["Y"]) and torch.equal(bd["Z_f"], a["Z"]) and torch.equal(bd["Z_b"], f2["Z"])
    # state hand-off: continuing from W_T1 over the rest equals the whole run
    T1 = 96 if wl.T > 96 else wl.T // 2 + 1
    first = _lib.forward(_cfg(wl, algo, T=T1), dev["X"][:, :T1].contiguous(), dev["theta"], dev["W1_0"],
                         dev["W2_0"], dev["alpha_f"], want_z=True, want_state=True)
    rest = _lib.forward(_cfg(wl, algo, T=wl.T - T1), dev["X"][:, T1:].contiguous(), dev["theta"],
                        first["W1_T"][0].contiguous(), first["W2_T"][0].contiguous(), dev["alpha_f"], want_z=True,
                        want_state=True)
    torch.cuda.synchronize()
    whole = [(torch.cat([first["Z"], rest["Z"]], 1), a["Z"]), (rest["W1_T"], a["W1_T"]), (rest["W2_T"], a["W2_T"])]
    if algo != "coop":
        for got, want in whole:
            assert torch.equal(got, want)
    else:
        # the cooperative scan applies each token's W1 update one token late (the next
        # pre-activation is k W1 before the update plus its rank-1 correction), so a run
        # continued from W_T1 rounds its first pre-activation differently: equal to fp32
        # rounding
        for got, want in whole:
            err = (got - want).abs().max().item()
            assert err <= 1e-5 * want.abs().max().item(), err
    # a call that ran to the end reports that its cooperative scan did not stop early
    ws = _lib._workspace(cfg, True, dev["X"])
    _lib.bidir(cfg, dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"], dev["alpha_b"], workspace=ws)
    assert not _lib.coop_aborted(cfg, True, ws)


# ----------------------------------------------------------------------------
# the five layer configurations at full size
# ----------------------------------------------------------------------------

def test_tiny_f32_full_config():
    wl = W.WORKLOADS["tiny_f32"]
    print("[config] tiny_f32 full", flush=True)
    inp = W.make_inputs(wl)
    got = _gpu_forward(wl, device_inputs(wl, inp), "auto")
    ref = _oracle_forward(wl, f64_inputs(wl, inp))
    _check_forward(wl, got, ref)


def test_seg14k_full_config_all_heads():
    wl = W.WORKLOADS["seg14k"]
    print("[config] seg14k full, all heads", flush=True)
    inp = W.make_inputs(wl)
    got = _gpu_forward(wl, device_inputs(wl, inp), "auto")
    ref = _oracle_forward(wl, f64_inputs(wl, inp))
    _check_forward(wl, got, ref)
    ten = rel_l2_tenths(from_device(got["Z"]), ref["Z"])
    print("  Z rel-L2 per tenth:", " ".join(f"{e:.1e}" for e in ten), flush=True)
    assert max(ten) <= BF16_TOL, ten


def test_many_chains_project_then_scan():
    """Four sequences of 48 heads (192 scan chains): too few CUs are left beside the
    scan, so each direction projects all its tokens on the whole chip and then scans
    (one chunk per direction).  Against the oracle, every head."""
    wl = W.WORKLOADS["batch4x76k"].replace(T=300, seg_len=0, alpha_f=0.1, alpha_b=0.2, name="batch4_small")
    print(f"[many chains] B{wl.B} T{wl.T} H{wl.H}", flush=True)
    inp = W.make_inputs(wl)
    got = _gpu_bidir(wl, device_inputs(wl, inp), "mfma")
    f64 = f64_inputs(wl, inp)
    ref = O.ttt_bidir(f64["X"], f64["theta"], f64["W1_0"], f64["W2_0"], f64["alpha_f"], f64["alpha_b"],
                      eta=wl.eta, b=wl.b, loss=wl.loss, gelu_form=wl.gelu, workers=workers())
    _check("Y", from_device(got["Y"]), ref["Y"], wl.io_dtype)
    _check("Z_f", from_device(got["Z_f"]), ref["Z_f"], wl.io_dtype)
    _check("Z_b", from_device(got["Z_b"]), ref["Z_b"], wl.io_dtype)
