"""ttt_mlp_bidir_noalloc, the bidirectional layer on the library's static
workspace, against ttt_mlp_bidir with a caller workspace, through the C ABI.

The two calls run the same kernels on the same inputs, so their outputs must
agree bit for bit (stricter than the oracle tolerances).  Two calls in a row,
the second smaller, so that the second runs on what the first left in the
shared array; then a call whose device memory use is measured around the bare
C call: it must not change the free device memory.
"""
import ctypes

import pytest

from test_rnn_layer_amd import workloads as W

from tests._common import device_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# first a multi-launch MFMA case (2,003 tokens: four scan chunks per direction, ragged tail),
# then a smaller one (fewer heads' worth of workspace, one chunk)
CALLS = [
    W.WORKLOADS["seg14k"].replace(T=2003, H=2, alpha_b=0.2, name="noalloc_chunks"),
    W.WORKLOADS["seg14k"].replace(T=300, H=1, alpha_b=0.2, name="noalloc_small"),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from test_rnn_layer_amd import _lib
    _lib.lib()  # the HIP library must load: no fallback
    yield


def _cfg(wl, algo="auto"):
    from test_rnn_layer_amd import _lib
    return _lib.make_config(wl.B, wl.T, wl.H, wl.d, wl.m, wl.b, wl.eta, io_dtype=wl.io_dtype, algo=algo)


def _same(a, b):
    for k in a:
        if a[k] is None:
            assert b[k] is None, k
            continue
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("algo", ["auto", "generic"])
def test_noalloc_matches_bidir_twice(algo):
    from test_rnn_layer_amd import _lib
    for wl in CALLS:
        print(f"[noalloc] {wl.name} algo={algo} T={wl.T} H={wl.H}", flush=True)
        dev = device_inputs(wl, W.make_inputs(wl))
        cfg = _cfg(wl, algo)
        ref = _lib.bidir(cfg, dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"], dev["alpha_b"],
                         want_z=True, want_state=True)
        got = _lib.bidir_noalloc(cfg, dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"],
                                 dev["alpha_b"], want_z=True, want_state=True)
        torch.cuda.synchronize()
        _same(got, ref)


def test_noalloc_allocates_nothing():
    from test_rnn_layer_amd import _lib
    wl = CALLS[1]
    dev = device_inputs(wl, W.make_inputs(wl))
    cfg = _cfg(wl)
    first = _lib.bidir_noalloc(cfg, dev["X"], dev["theta"], dev["W1_0"], dev["W2_0"], dev["alpha_f"], dev["alpha_b"])
    Y = torch.empty_like(dev["X"])
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    st = _lib.lib().ttt_mlp_bidir_noalloc(ctypes.byref(cfg), dev["X"].data_ptr(), dev["theta"].data_ptr(),
                                          dev["W1_0"].data_ptr(), dev["W2_0"].data_ptr(), dev["alpha_f"].data_ptr(),
                                          dev["alpha_b"].data_ptr(), Y.data_ptr(), None, None, None, None, None,
                                          None, stream)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert st == _lib.TTT_OK, _lib.lib().ttt_mlp_last_error()
    assert free1 == free0, (free0, free1)
    assert torch.equal(Y, first["Y"])
