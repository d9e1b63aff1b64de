"""Oracle parity of the three long bidirectional configurations at full length.

bidir100k (100,800 tokens), bidir307k (307,200 tokens with per-segment mean
shifts) and bigstate307k (307,200 tokens, d = 128, b = 1) run once through
ttt_mlp_bidir in the launch configuration the benchmark times.  The fp64
oracle then runs the same layer from the same seeded inputs:

* forward pass: every head over the whole sequence.  Its gated output X' is
  the reversed pass's input, and theta mixes every channel, so the reversed
  pass of any head needs the forward pass of all of them.  The oracle keeps X'
  in float64; the library stores it in bf16 (its only rounding of X').
* reversed pass: every head at bidir100k; the first and the last head at the
  two 307,200-token configurations.

Compared (relative L2 <= 2e-2, the bar for bf16-input paths), over the whole
sequence and separately in each tenth of it (late tokens are smaller, and a
whole-sequence norm is dominated by the early ones): Z of each direction, X',
the layer output Y, and the final states of both passes.

The oracle takes minutes here; each head group prints a progress line.
"""
import time

import numpy as np
import pytest

from oracle import ttt_oracle as O
from test_rnn_layer_amd import workloads as W

from tests._common import (TenthsError, device_inputs, f64_inputs, head_cols, host_f32, rel_l2, workers)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2

# name -> heads whose reversed pass the oracle runs (None: all)
FULL = {"bidir100k": None, "bidir307k": "ends", "bigstate307k": "ends"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from test_rnn_layer_amd import _lib
    _lib.lib()  # the HIP library must load: no fallback
    yield


@pytest.fixture
def say(capsys):
    """Prints past pytest's output capture: the oracle runs for minutes, and a
    run that prints nothing for that long looks hung."""
    def _say(msg):
        with capsys.disabled():
            print(msg, flush=True)
    return _say


def _report(say, name, acc, tol=BF16_TOL):
    ten = acc.tenths()
    say(f"  {name}: rel-L2 {acc.overall():.2e}; per tenth " + " ".join(f"{e:.1e}" for e in ten))
    assert acc.overall() <= tol, (name, acc.overall())
    assert max(ten) <= tol, (name, ten)


def _check_state(say, name, got, ref):
    err = rel_l2(got, ref)
    say(f"  {name}: rel-L2 {err:.2e}")
    assert err <= BF16_TOL, (name, err)


def _groups(heads, size):
    return [heads[i:i + size] for i in range(0, len(heads), size)]


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", list(FULL))
def test_full_length_bidir_matches_oracle(name, say):
    from test_rnn_layer_amd import _lib
    wl = W.WORKLOADS[name]
    H, d, T = wl.H, wl.d, wl.T
    rev_heads = list(range(H)) if FULL[name] is None else [0, H - 1]
    rcols = head_cols(rev_heads, d)
    say(f"[full length] {name}: B{wl.B} T{T} H{H} d{d} m{wl.m} b{wl.b}; reversed pass checked on heads "
        f"{'all' if FULL[name] is None else rev_heads}")
    t0 = time.perf_counter()
    inp = W.make_inputs(wl)
    dev = device_inputs(wl, inp)
    cfg = _lib.make_config(wl.B, T, H, d, wl.m, wl.b, wl.eta, io_dtype=wl.io_dtype)
    algo = _lib.select_algo(cfg)
    r = _lib.bidir(cfg, dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"], dev["alpha_b"],
                   want_z=True, want_state=True)
    f = _lib.forward(cfg, dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"])
    torch.cuda.synchronize()
    # the reversed pass of the library's own X' gives the bidirectional output bit for bit
    g = _lib.forward(cfg, f["Y"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_b"], reverse=True)
    torch.cuda.synchronize()
    assert torch.equal(g["Y"], r["Y"])
    del g
    gpu = dict(Zf=host_f32(r["Z_f"]), Xp=host_f32(f["Y"]), Zb=host_f32(r["Z_b"], rcols),
               Y=host_f32(r["Y"], rcols))
    state = {k: r[k][:, rev_heads].cpu().numpy() if k.endswith("b") else r[k].cpu().numpy()
             for k in ("W1_Tf", "W2_Tf", "W1_Tb", "W2_Tb")}
    del r, f, dev
    torch.cuda.empty_cache()
    say(f"  GPU ({algo}) done, outputs on the host: {time.perf_counter() - t0:.1f} s")
    for k in ("Zf", "Zb", "Xp"):
        assert np.isfinite(gpu[k]).all(), k

    f64 = f64_inputs(wl, inp)
    del inp
    nw = workers()
    kw = dict(eta=wl.eta, b=wl.b, loss=wl.loss, gelu_form=wl.gelu, workers=nw)

    # forward pass, every head, in groups of as many heads as worker processes
    Xp = np.empty((wl.B, T, wl.D))
    err_zf, err_xp = TenthsError(T), TenthsError(T)
    for grp in _groups(list(range(H)), nw):
        cols = head_cols(grp, d)
        o = O.ttt_forward(f64["X"], f64["theta"], f64["W1_0"], f64["W2_0"], f64["alpha_f"], heads=grp, **kw)
        Xp[..., cols] = o["Y"]
        err_zf.add(gpu["Zf"][..., cols], o["Z"])
        err_xp.add(gpu["Xp"][..., cols], o["Y"])
        _check_state(say, f"W1_Tf heads {grp[0]}-{grp[-1]}", state["W1_Tf"][:, grp], o["W1_T"])
        _check_state(say, f"W2_Tf heads {grp[0]}-{grp[-1]}", state["W2_Tf"][:, grp], o["W2_T"])
        say(f"  oracle forward, heads {grp[0]}-{grp[-1]}: {time.perf_counter() - t0:.1f} s")
    del gpu["Zf"], gpu["Xp"]
    _report(say, "Z_f (every head)", err_zf)
    _report(say, "X' (every head)", err_xp)

    # reversed pass over the oracle's X'
    err_zb, err_y = TenthsError(T), TenthsError(T)
    w1b, w2b = [], []
    for grp in _groups(rev_heads, nw):
        idx = [rev_heads.index(h) for h in grp]
        sub = head_cols(idx, d)
        o = O.ttt_forward(Xp, f64["theta"], f64["W1_0"], f64["W2_0"], f64["alpha_b"], reverse=True, heads=grp, **kw)
        err_zb.add(gpu["Zb"][..., sub], o["Z"])
        err_y.add(gpu["Y"][..., sub], o["Y"])
        w1b.append(o["W1_T"])
        w2b.append(o["W2_T"])
        say(f"  oracle reversed pass, heads {grp[0]}-{grp[-1]}: {time.perf_counter() - t0:.1f} s")
    _report(say, "Z_b", err_zb)
    _report(say, "Y", err_y)
    _check_state(say, "W1_Tb", state["W1_Tb"], np.concatenate(w1b, axis=1))
    _check_state(say, "W2_Tb", state["W2_Tb"], np.concatenate(w2b, axis=1))
