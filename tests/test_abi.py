"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments on the host before touching a device (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

from test_rnn_layer_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ttt_mlp.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ttt_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("ttt_mlp_forward", "ttt_mlp_bidir", "ttt_mlp_workspace_size", "ttt_mlp_status_string"):
        assert n in names
    assert sorted(L.EXPORTED) == names


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert lib.ttt_mlp_version() >> 16 == 1


def test_config_struct_layout_matches_header(tmp_path):
    # int64 B, T; int32 H, d, m, b; float eta; int32 loss, gelu, io_dtype, algo, model
    assert ctypes.sizeof(L.Config) == 56
    assert L.Config.eta.offset == 32 and L.Config.algo.offset == 48 and L.Config.model.offset == 52
    # the C compiler's view of the header agrees with the binding
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "ttt_mlp.h"\n'
                   "int main(void) { printf(\"%zu %zu %zu %zu\\n\", sizeof(ttt_mlp_config), "
                   "offsetof(ttt_mlp_config, eta), offsetof(ttt_mlp_config, algo), offsetof(ttt_mlp_config, model)); "
                   "return 0; }\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    assert [int(x) for x in out] == [ctypes.sizeof(L.Config), L.Config.eta.offset, L.Config.algo.offset,
                                     L.Config.model.offset]


def test_status_strings():
    for s in (0, -1, -2, -3, -4):
        assert L.status_string(s)
    assert L.status_string(-99) == "unknown status"


def cfg(**kw):
    base = dict(B=1, T=64, H=2, d=64, m=256, b=16, eta=0.1 / 16)
    base.update(kw)
    return L.make_config(**base)


def test_workspace_size_and_validation():
    # generic: fp32 Q, K, V plus the fp32 state; MFMA: bf16 Q, K, V token blocks (4 per 64 tokens)
    assert L.workspace_size(cfg(algo="generic"), False) >= 3 * 2 * 64 * 64 * 4 + 2 * 2 * 64 * 256 * 4
    assert L.workspace_size(cfg(algo="mfma"), False) >= 2 * 4 * 3 * 16 * 64 * 2
    assert L.workspace_size(cfg(T=0), True) > 0
    bad = [dict(B=0), dict(T=-1), dict(H=0), dict(d=0), dict(b=0), dict(eta=-1.0), dict(eta=float("nan"))]
    for kw in bad:
        with pytest.raises(L.TTTError) as e:
            L.workspace_size(cfg(**kw), False)
        assert e.value.status == L.TTT_ERR_INVALID_ARG
    c = cfg()
    c.loss = 7
    with pytest.raises(L.TTTError) as e:
        L.workspace_size(c, False)
    assert e.value.status == L.TTT_ERR_INVALID_ARG
    # a mini-batch working set beyond the generic kernel's LDS budget
    with pytest.raises(L.TTTError) as e:
        L.workspace_size(cfg(b=64, m=512, d=128), False)
    assert e.value.status == L.TTT_ERR_UNSUPPORTED


def test_compute_calls_reject_bad_pointers_on_the_host():
    lib = L.lib()
    c = cfg()
    n = L.workspace_size(c, False)
    fake = 1 << 40  # never dereferenced: every call below fails its host checks first
    st = lib.ttt_mlp_forward(ctypes.byref(c), None, fake, fake, fake, fake, 0, fake, None, None, None, fake, n, None)
    assert st == L.TTT_ERR_INVALID_ARG
    st = lib.ttt_mlp_forward(ctypes.byref(c), fake, fake, fake, fake, fake, 0, fake + 4096, None, None, None,
                             fake + (1 << 30), n - 1, None)
    assert st == L.TTT_ERR_WORKSPACE
    # Y overlapping X
    st = lib.ttt_mlp_forward(ctypes.byref(c), fake, fake + (1 << 32), fake + (2 << 32), fake + (3 << 32),
                             fake + (4 << 32), 0, fake + 64, None, None, None, fake + (5 << 32), n, None)
    assert st == L.TTT_ERR_INVALID_ARG and b"overlaps" in lib.ttt_mlp_last_error()
    st = lib.ttt_mlp_forward(ctypes.byref(c), fake, fake, fake, fake, fake, 2, fake, None, None, None, fake, n, None)
    assert st == L.TTT_ERR_INVALID_ARG
    st = lib.ttt_mlp_bidir(ctypes.byref(c), fake, fake, fake, fake, fake, None, fake, None, None, None, None,
                           None, None, fake, n, None)
    assert st == L.TTT_ERR_INVALID_ARG
    st = lib.ttt_mlp_kernel_timing(5, ctypes.byref(ctypes.c_double()), ctypes.byref(ctypes.c_int64()))
    assert st == L.TTT_ERR_INVALID_ARG


def test_noalloc_rejects_a_workspace_beyond_the_static_array_on_the_host():
    lib = L.lib()
    fake = 1 << 40  # never dereferenced: the size check comes first
    limit = 320 << 20
    # one 3-second segment (14,400 tokens, 48 heads of width 64) fits the array; 20,000 tokens do not
    assert L.workspace_size(cfg(H=48, T=14_400), True) <= limit
    big = cfg(H=48, T=20_000)
    assert L.workspace_size(big, True) > limit
    st = lib.ttt_mlp_bidir_noalloc(ctypes.byref(big), fake, fake + (1 << 34), fake + (2 << 34), fake + (3 << 34),
                                   fake + (4 << 34), fake + (5 << 34), fake + (6 << 34), None, None, None, None, None,
                                   None, None)
    assert st == L.TTT_ERR_WORKSPACE and b"static workspace" in lib.ttt_mlp_last_error()
    st = lib.ttt_mlp_bidir_noalloc(ctypes.byref(cfg(b=0)), fake, fake, fake, fake, fake, fake, fake, None, None, None,
                                   None, None, None, None)
    assert st == L.TTT_ERR_INVALID_ARG


def test_coop_aborted_query_on_the_host():
    lib = L.lib()
    v = ctypes.c_int32(7)
    # a configuration that runs another scan: nothing is read, the answer is "no"
    assert lib.ttt_mlp_coop_aborted(ctypes.byref(cfg()), 1, None, 0, None, ctypes.byref(v)) == L.TTT_OK
    assert v.value == 0
    big = cfg(d=128, m=512, b=1, eta=0.05, algo="coop")
    assert lib.ttt_mlp_coop_aborted(ctypes.byref(big), 1, None, 0, None, ctypes.byref(v)) == L.TTT_ERR_WORKSPACE
    assert lib.ttt_mlp_coop_aborted(ctypes.byref(big), 1, 1 << 40, 1, None, ctypes.byref(v)) == L.TTT_ERR_WORKSPACE
    assert lib.ttt_mlp_coop_aborted(ctypes.byref(big), 2, None, 0, None, ctypes.byref(v)) == L.TTT_ERR_INVALID_ARG
    assert lib.ttt_mlp_coop_aborted(ctypes.byref(big), 1, None, 0, None, None) == L.TTT_ERR_INVALID_ARG


def test_algo_selection():
    assert L.select_algo(cfg()) == "mfma"
    assert L.select_algo(cfg(algo="generic")) == "generic"
    assert L.select_algo(L.make_config(1, 10, 1, 16, 64, 1, 0.1, io_dtype="f32")) == "generic"
    # the MFMA scan indexes token rows with 32-bit integers: longer sequences use the generic scan
    assert L.select_algo(cfg(T=(1 << 31) - 1)) == "mfma"
    assert L.select_algo(cfg(T=1 << 31)) == "generic"
    with pytest.raises(L.TTTError) as e:
        L.select_algo(cfg(b=8, algo="mfma"))
    assert e.value.status == L.TTT_ERR_UNSUPPORTED
    # the per-token large-state shape goes to the cooperative scan, in any io dtype and GELU form
    big = dict(B=1, T=10, H=2, d=128, m=512, b=1, eta=0.05)
    assert L.select_algo(L.make_config(**big)) == "coop"
    assert L.select_algo(L.make_config(**big, io_dtype="f32", gelu="tanh")) == "coop"
    assert L.select_algo(L.make_config(**big, algo="generic")) == "generic"
    with pytest.raises(L.TTTError) as e:
        L.select_algo(L.make_config(**dict(big, b=2), algo="coop"))
    assert e.value.status == L.TTT_ERR_UNSUPPORTED
    # coop workspace: fp32 Q, K, V plus the exchange slots (2 parities x 8 workgroups x 256 entries x 8 B per head)
    assert L.workspace_size(L.make_config(**big), False) >= 3 * 2 * 10 * 128 * 4 + 2 * 2 * 8 * 256 * 8


def test_linear_model_selection_and_validation():
    lin = dict(B=1, T=100, H=3, d=64, m=64, b=16, eta=0.1 / 16, model="linear")
    assert L.select_algo(L.make_config(**lin)) == "mfma"
    assert L.select_algo(L.make_config(**lin, io_dtype="f32")) == "generic"
    assert L.select_algo(L.make_config(**dict(lin, b=4))) == "generic"
    assert L.select_algo(L.make_config(**lin, algo="generic")) == "generic"
    # the tanh GELU switch does not concern the linear model
    assert L.select_algo(L.make_config(**lin, gelu="tanh")) == "mfma"
    for bad in (dict(lin, m=256), dict(lin, d=32, m=64)):
        with pytest.raises(L.TTTError) as e:
            L.workspace_size(L.make_config(**bad), False)
        assert e.value.status == L.TTT_ERR_INVALID_ARG
    with pytest.raises(L.TTTError) as e:
        L.select_algo(L.make_config(**dict(lin, d=128, m=128, b=1), algo="coop"))
    assert e.value.status == L.TTT_ERR_UNSUPPORTED
    c = L.make_config(**lin)
    c.model = 5
    with pytest.raises(L.TTTError) as e:
        L.workspace_size(c, False)
    assert e.value.status == L.TTT_ERR_INVALID_ARG
    # workspace: bf16 Q, K, V token blocks plus one d x d state per head
    assert L.workspace_size(L.make_config(**lin), True) >= 3 * 7 * 3 * 16 * 64 * 2 + 3 * 64 * 64 * 4
    # W2_0 may be NULL for the linear model (the host checks pass it; a NULL W1_0 is refused)
    lib = L.lib()
    n = L.workspace_size(c.__class__(**{f: getattr(L.make_config(**lin), f) for f, _ in L.Config._fields_}), False)
    fake = 1 << 40
    cl = L.make_config(**lin)
    st = lib.ttt_mlp_forward(ctypes.byref(cl), fake, fake + (1 << 32), None, None, fake + (2 << 32), 0,
                             fake + (3 << 32), None, None, None, fake + (4 << 32), n, None)
    assert st == L.TTT_ERR_INVALID_ARG and b"W1_0" in lib.ttt_mlp_last_error()


def test_backward_workspace_and_validation():
    c = cfg(algo="auto")
    one, two = L.backward_workspace_size(c, False), L.backward_workspace_size(c, True)
    # at least Q/K/V and their gradients in fp32, Z, and one checkpoint per direction
    assert one >= 2 * 3 * 64 * 128 * 4 + 64 * 128 * 4 + 2 * 2 * 64 * 256 * 4
    assert two > one
    assert L.backward_workspace_size(cfg(T=0), True) > 0
    for bad, status in [(dict(model="linear", m=64), L.TTT_ERR_UNSUPPORTED), (dict(algo="mfma"), L.TTT_ERR_UNSUPPORTED),
                        (dict(b=64, m=512, d=128), L.TTT_ERR_UNSUPPORTED), (dict(eta=-1.0), L.TTT_ERR_INVALID_ARG)]:
        with pytest.raises(L.TTTError) as e:
            L.backward_workspace_size(cfg(**bad), False)
        assert e.value.status == status, bad
    lib = L.lib()
    n = L.backward_workspace_size(c, False)
    fake = 1 << 40  # never dereferenced: the host checks fail first
    f = lambda k: fake + (k << 32)
    st = lib.ttt_mlp_backward(ctypes.byref(c), f(0), f(1), f(2), f(3), f(4), 0, None, f(5), f(6), f(7), f(8), f(9),
                              f(10), n, None)
    assert st == L.TTT_ERR_INVALID_ARG  # dY missing
    st = lib.ttt_mlp_backward(ctypes.byref(c), f(0), f(1), f(2), f(3), f(4), 0, f(11), f(5), f(6), f(7), f(8), f(9),
                              f(10), n - 1, None)
    assert st == L.TTT_ERR_WORKSPACE
    st = lib.ttt_mlp_backward(ctypes.byref(c), f(0), f(1), f(2), f(3), f(4), 0, f(11), f(11) + 64, f(6), f(7), f(8),
                              f(9), f(10), n, None)
    assert st == L.TTT_ERR_INVALID_ARG and b"overlaps" in lib.ttt_mlp_last_error()  # dX over dY
    n2 = L.backward_workspace_size(c, True)
    st = lib.ttt_mlp_bidir_backward(ctypes.byref(c), f(0), f(1), f(2), f(3), f(4), None, f(11), f(5), f(6), f(7),
                                    f(8), f(9), f(12), f(10), n2, None)
    assert st == L.TTT_ERR_INVALID_ARG  # alpha_b missing


def test_attention_and_hybrid_validation():
    lib = L.lib()
    c = cfg()
    assert L.hybrid_workspace_size(c, 14400) > L.workspace_size(c, True)
    for bad, status in [(dict(io_dtype="f32"), L.TTT_ERR_UNSUPPORTED), (dict(d=32, m=128), L.TTT_ERR_UNSUPPORTED)]:
        with pytest.raises(L.TTTError) as e:
            L.hybrid_workspace_size(cfg(**bad), 100)
        assert e.value.status == status, bad
    with pytest.raises(L.TTTError) as e:
        L.hybrid_workspace_size(c, 0)
    assert e.value.status == L.TTT_ERR_INVALID_ARG
    fake = 1 << 40
    st = lib.ttt_segment_attention(ctypes.byref(c), 16, fake, None, None)
    assert st == L.TTT_ERR_INVALID_ARG
    st = lib.ttt_segment_attention(ctypes.byref(c), 16, fake, fake + 64, None)  # O over QKV
    assert st == L.TTT_ERR_INVALID_ARG and b"overlaps" in lib.ttt_mlp_last_error()
