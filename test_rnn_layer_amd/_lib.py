"""Thin ctypes binding of libttt_mlp.so (the C ABI declared in include/ttt_mlp.h).

Only argument marshalling lives here: torch supplies device memory (outputs
and workspace are allocated with torch.empty on the input's device) and the
current HIP stream; every arithmetic step runs in the library's kernels.  If
the library is missing, loading raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libttt_mlp.so")

TTT_OK, TTT_ERR_INVALID_ARG, TTT_ERR_UNSUPPORTED, TTT_ERR_WORKSPACE, TTT_ERR_HIP = 0, -1, -2, -3, -4
TTT_F32, TTT_BF16 = 0, 1
TTT_LOSS_MEAN, TTT_LOSS_SUM = 0, 1
TTT_GELU_ERF, TTT_GELU_TANH = 0, 1
TTT_MODEL_MLP, TTT_MODEL_LINEAR = 0, 1
TTT_ALGO_AUTO, TTT_ALGO_GENERIC, TTT_ALGO_MFMA, TTT_ALGO_COOP = 0, 1, 2, 3
TTT_KERNEL_PROJECT, TTT_KERNEL_SCAN, TTT_KERNEL_BACKWARD, TTT_KERNEL_GRAD_GEMM, TTT_KERNEL_ATTENTION = 0, 1, 2, 3, 4

EXPORTED = [
    "ttt_mlp_version", "ttt_mlp_status_string", "ttt_mlp_last_error", "ttt_mlp_workspace_size",
    "ttt_mlp_select_algo",
    "ttt_mlp_forward", "ttt_mlp_bidir", "ttt_mlp_bidir_noalloc", "ttt_mlp_coop_aborted", "ttt_mlp_project", "ttt_mlp_set_kernel_timing",
    "ttt_mlp_kernel_timing", "ttt_mlp_reset_kernel_timing",
    "ttt_mlp_backward_workspace_size", "ttt_mlp_backward", "ttt_mlp_bidir_backward",
    "ttt_segment_attention", "ttt_hybrid_block_workspace_size", "ttt_hybrid_block",
]


class Config(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("T", ctypes.c_int64),
        ("H", ctypes.c_int32), ("d", ctypes.c_int32), ("m", ctypes.c_int32), ("b", ctypes.c_int32),
        ("eta", ctypes.c_float),
        ("loss", ctypes.c_int32), ("gelu", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
        ("algo", ctypes.c_int32), ("model", ctypes.c_int32),
    ]


class TTTError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_string(status)} ({status}): {detail}")
        self.status = status


_lib = None
_vp, _fp, _i32, _sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t


def use_library(path: str):
    """Load the library from `path` instead (the phase-marks measurement build);
    only before the first call that loads it."""
    global LIB_PATH
    if _lib is not None and os.path.abspath(path) != LIB_PATH:
        raise RuntimeError(f"{LIB_PATH} is already loaded")
    LIB_PATH = os.path.abspath(path)


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m test_rnn_layer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.ttt_mlp_version.restype = _i32
        L.ttt_mlp_status_string.restype = ctypes.c_char_p
        L.ttt_mlp_status_string.argtypes = [_i32]
        L.ttt_mlp_last_error.restype = ctypes.c_char_p
        L.ttt_mlp_workspace_size.restype = _i32
        L.ttt_mlp_workspace_size.argtypes = [ctypes.POINTER(Config), _i32, ctypes.POINTER(_sz)]
        L.ttt_mlp_select_algo.restype = _i32
        L.ttt_mlp_select_algo.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(_i32)]
        L.ttt_mlp_forward.restype = _i32
        L.ttt_mlp_forward.argtypes = [ctypes.POINTER(Config), _vp, _vp, _fp, _fp, _fp, _i32,
                                      _vp, _fp, _fp, _fp, _vp, _sz, _vp]
        L.ttt_mlp_bidir.restype = _i32
        L.ttt_mlp_bidir.argtypes = [ctypes.POINTER(Config), _vp, _vp, _fp, _fp, _fp, _fp,
                                    _vp, _fp, _fp, _fp, _fp, _fp, _fp, _vp, _sz, _vp]
        L.ttt_mlp_bidir_noalloc.restype = _i32
        L.ttt_mlp_bidir_noalloc.argtypes = [ctypes.POINTER(Config), _vp, _vp, _fp, _fp, _fp, _fp,
                                            _vp, _fp, _fp, _fp, _fp, _fp, _fp, _vp]
        L.ttt_mlp_coop_aborted.restype = _i32
        L.ttt_mlp_coop_aborted.argtypes = [ctypes.POINTER(Config), _i32, _vp, _sz, _vp, ctypes.POINTER(_i32)]
        L.ttt_mlp_project.restype = _i32
        L.ttt_mlp_project.argtypes = [ctypes.POINTER(Config), _vp, _vp, _fp, _vp]
        L.ttt_mlp_set_kernel_timing.restype = _i32
        L.ttt_mlp_set_kernel_timing.argtypes = [_i32]
        L.ttt_mlp_kernel_timing.restype = _i32
        L.ttt_mlp_kernel_timing.argtypes = [_i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
        L.ttt_mlp_reset_kernel_timing.restype = _i32
        L.ttt_mlp_backward_workspace_size.restype = _i32
        L.ttt_mlp_backward_workspace_size.argtypes = [ctypes.POINTER(Config), _i32, ctypes.POINTER(_sz)]
        L.ttt_mlp_backward.restype = _i32
        L.ttt_mlp_backward.argtypes = [ctypes.POINTER(Config), _vp, _vp, _fp, _fp, _fp, _i32, _fp,
                                       _fp, _fp, _fp, _fp, _fp, _vp, _sz, _vp]
        L.ttt_mlp_bidir_backward.restype = _i32
        L.ttt_mlp_bidir_backward.argtypes = [ctypes.POINTER(Config), _vp, _vp, _fp, _fp, _fp, _fp, _fp,
                                             _fp, _fp, _fp, _fp, _fp, _fp, _vp, _sz, _vp]
        L.ttt_segment_attention.restype = _i32
        L.ttt_segment_attention.argtypes = [ctypes.POINTER(Config), ctypes.c_int64, _vp, _vp, _vp]
        L.ttt_hybrid_block_workspace_size.restype = _i32
        L.ttt_hybrid_block_workspace_size.argtypes = [ctypes.POINTER(Config), ctypes.c_int64, ctypes.POINTER(_sz)]
        L.ttt_hybrid_block.restype = _i32
        L.ttt_hybrid_block.argtypes = [ctypes.POINTER(Config), ctypes.c_int64, _vp, _vp, _vp, _vp, _fp, _fp, _fp, _fp,
                                       _vp, _vp, _sz, _vp]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().ttt_mlp_status_string(status).decode()


def _check(status: int):
    if status != TTT_OK:
        raise TTTError(status, lib().ttt_mlp_last_error().decode())


def make_config(B, T, H, d, m, b, eta, *, io_dtype="bf16", loss="mean", gelu="erf", algo="auto",
                model="mlp") -> Config:
    return Config(B=B, T=T, H=H, d=d, m=m, b=b, eta=eta,
                  model={"mlp": TTT_MODEL_MLP, "linear": TTT_MODEL_LINEAR}[model],
                  loss={"mean": TTT_LOSS_MEAN, "sum": TTT_LOSS_SUM}[loss],
                  gelu={"erf": TTT_GELU_ERF, "tanh": TTT_GELU_TANH}[gelu],
                  io_dtype={"f32": TTT_F32, "bf16": TTT_BF16}[io_dtype],
                  algo={"auto": TTT_ALGO_AUTO, "generic": TTT_ALGO_GENERIC, "mfma": TTT_ALGO_MFMA,
                        "coop": TTT_ALGO_COOP}[algo])


def workspace_size(cfg: Config, bidir: bool) -> int:
    n = _sz(0)
    _check(lib().ttt_mlp_workspace_size(ctypes.byref(cfg), int(bidir), ctypes.byref(n)))
    return n.value


def select_algo(cfg: Config) -> str:
    """The scan kernel a call with cfg runs: "generic" or "mfma"."""
    a = _i32(0)
    _check(lib().ttt_mlp_select_algo(ctypes.byref(cfg), ctypes.byref(a)))
    return {TTT_ALGO_GENERIC: "generic", TTT_ALGO_MFMA: "mfma", TTT_ALGO_COOP: "coop"}[a.value]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _state_out(cfg, like):
    """Final-state outputs: W1_T, W2_T (the linear model has only W = W1, [B, H, d, d])."""
    import torch
    kw = dict(dtype=torch.float32, device=like.device)
    w1 = torch.empty((cfg.B, cfg.H, cfg.d, cfg.m), **kw)
    return (w1, None) if cfg.model == TTT_MODEL_LINEAR else (w1, torch.empty((cfg.B, cfg.H, cfg.m, cfg.d), **kw))


def _workspace(cfg, bidir, like):
    import torch
    return torch.empty(max(workspace_size(cfg, bidir), 1), dtype=torch.uint8, device=like.device)


def forward(cfg: Config, X, theta, W1_0, W2_0, alpha, *, reverse=False, want_z=False, want_state=False,
            workspace=None):
    """ttt_mlp_forward.  Returns dict(Y, Z?, W1_T?, W2_T?)."""
    import torch
    Y = torch.empty_like(X)
    Z = torch.empty(X.shape, dtype=torch.float32, device=X.device) if want_z else None
    W1T, W2T = _state_out(cfg, X) if want_state else (None, None)
    ws = _workspace(cfg, False, X) if workspace is None else workspace
    _check(lib().ttt_mlp_forward(ctypes.byref(cfg), _ptr(X), _ptr(theta), _ptr(W1_0), _ptr(W2_0), _ptr(alpha),
                                 int(reverse), _ptr(Y), _ptr(Z), _ptr(W1T), _ptr(W2T), _ptr(ws), ws.numel(),
                                 _stream(X.device)))
    return dict(Y=Y, Z=Z, W1_T=W1T, W2_T=W2T)


def bidir(cfg: Config, X, theta, W1_0, W2_0, alpha_f, alpha_b, *, want_z=False, want_state=False,
          workspace=None, out=None):
    """ttt_mlp_bidir.  Returns dict(Y, Z_f?, Z_b?, W1_Tf?, W2_Tf?, W1_Tb?, W2_Tb?)."""
    import torch
    Y = torch.empty_like(X) if out is None else out
    mk = lambda: torch.empty(X.shape, dtype=torch.float32, device=X.device)
    Zf, Zb = (mk(), mk()) if want_z else (None, None)
    (W1f, W2f), (W1b, W2b) = (_state_out(cfg, X), _state_out(cfg, X)) if want_state else ((None, None), (None, None))
    ws = _workspace(cfg, True, X) if workspace is None else workspace
    _check(lib().ttt_mlp_bidir(ctypes.byref(cfg), _ptr(X), _ptr(theta), _ptr(W1_0), _ptr(W2_0), _ptr(alpha_f),
                               _ptr(alpha_b), _ptr(Y), _ptr(Zf), _ptr(Zb), _ptr(W1f), _ptr(W2f), _ptr(W1b),
                               _ptr(W2b), _ptr(ws), ws.numel(), _stream(X.device)))
    return dict(Y=Y, Z_f=Zf, Z_b=Zb, W1_Tf=W1f, W2_Tf=W2f, W1_Tb=W1b, W2_Tb=W2b)


def bidir_noalloc(cfg: Config, X, theta, W1_0, W2_0, alpha_f, alpha_b, *, want_z=False, want_state=False, out=None):
    """ttt_mlp_bidir_noalloc (the library's static workspace).  Returns as bidir()."""
    import torch
    Y = torch.empty_like(X) if out is None else out
    mk = lambda: torch.empty(X.shape, dtype=torch.float32, device=X.device)
    Zf, Zb = (mk(), mk()) if want_z else (None, None)
    (W1f, W2f), (W1b, W2b) = (_state_out(cfg, X), _state_out(cfg, X)) if want_state else ((None, None), (None, None))
    _check(lib().ttt_mlp_bidir_noalloc(ctypes.byref(cfg), _ptr(X), _ptr(theta), _ptr(W1_0), _ptr(W2_0),
                                       _ptr(alpha_f), _ptr(alpha_b), _ptr(Y), _ptr(Zf), _ptr(Zb), _ptr(W1f),
                                       _ptr(W2f), _ptr(W1b), _ptr(W2b), _stream(X.device)))
    return dict(Y=Y, Z_f=Zf, Z_b=Zb, W1_Tf=W1f, W2_Tf=W2f, W1_Tb=W1b, W2_Tb=W2b)


def coop_aborted(cfg: Config, bidir: bool, workspace, device=None) -> bool:
    """ttt_mlp_coop_aborted: whether the cooperative scan of the last call on
    `workspace` stopped early (waits for the current stream)."""
    v = _i32(0)
    _check(lib().ttt_mlp_coop_aborted(ctypes.byref(cfg), int(bidir), _ptr(workspace),
                                      0 if workspace is None else workspace.numel(),
                                      _stream(device if workspace is None else workspace.device),
                                      ctypes.byref(v)))
    return bool(v.value)


def backward_workspace_size(cfg: Config, bidir: bool) -> int:
    n = _sz(0)
    _check(lib().ttt_mlp_backward_workspace_size(ctypes.byref(cfg), int(bidir), ctypes.byref(n)))
    return n.value


def _grad_outs(cfg, X):
    import torch
    kw = dict(dtype=torch.float32, device=X.device)
    D = cfg.H * cfg.d
    return dict(dX=torch.empty(X.shape, **kw), dtheta=torch.empty((3, D, D), **kw),
                dW1_0=torch.empty((cfg.H, cfg.d, cfg.m), **kw), dW2_0=torch.empty((cfg.H, cfg.m, cfg.d), **kw))


def backward(cfg: Config, X, theta, W1_0, W2_0, alpha, dY, *, reverse=False, workspace=None):
    """ttt_mlp_backward: gradients of sum(dY * Y) for one direction.
    Returns dict(dX, dtheta, dW1_0, dW2_0, dalpha), all fp32."""
    import torch
    g = _grad_outs(cfg, X)
    g["dalpha"] = torch.empty(alpha.shape, dtype=torch.float32, device=X.device)
    ws = (torch.empty(max(backward_workspace_size(cfg, False), 1), dtype=torch.uint8, device=X.device)
          if workspace is None else workspace)
    _check(lib().ttt_mlp_backward(ctypes.byref(cfg), _ptr(X), _ptr(theta), _ptr(W1_0), _ptr(W2_0), _ptr(alpha),
                                  int(reverse), _ptr(dY), _ptr(g["dX"]), _ptr(g["dtheta"]), _ptr(g["dW1_0"]),
                                  _ptr(g["dW2_0"]), _ptr(g["dalpha"]), _ptr(ws), ws.numel(), _stream(X.device)))
    return g


def bidir_backward(cfg: Config, X, theta, W1_0, W2_0, alpha_f, alpha_b, dY, *, workspace=None):
    """ttt_mlp_bidir_backward: gradients of sum(dY * Y) for the bidirectional layer.
    Returns dict(dX, dtheta, dW1_0, dW2_0, dalpha_f, dalpha_b), all fp32."""
    import torch
    g = _grad_outs(cfg, X)
    g["dalpha_f"] = torch.empty(alpha_f.shape, dtype=torch.float32, device=X.device)
    g["dalpha_b"] = torch.empty(alpha_b.shape, dtype=torch.float32, device=X.device)
    ws = (torch.empty(max(backward_workspace_size(cfg, True), 1), dtype=torch.uint8, device=X.device)
          if workspace is None else workspace)
    _check(lib().ttt_mlp_bidir_backward(ctypes.byref(cfg), _ptr(X), _ptr(theta), _ptr(W1_0), _ptr(W2_0),
                                        _ptr(alpha_f), _ptr(alpha_b), _ptr(dY), _ptr(g["dX"]), _ptr(g["dtheta"]),
                                        _ptr(g["dW1_0"]), _ptr(g["dW2_0"]), _ptr(g["dalpha_f"]),
                                        _ptr(g["dalpha_b"]), _ptr(ws), ws.numel(), _stream(X.device)))
    return g


def segment_attention(cfg: Config, seg_len: int, QKV):
    """ttt_segment_attention: QKV [B, T, 3 D] bf16 -> O [B, T, D] bf16."""
    import torch
    O = torch.empty((cfg.B, cfg.T, cfg.H * cfg.d), dtype=QKV.dtype, device=QKV.device)
    _check(lib().ttt_segment_attention(ctypes.byref(cfg), seg_len, _ptr(QKV), _ptr(O), _stream(QKV.device)))
    return O


def hybrid_workspace_size(cfg: Config, seg_len: int) -> int:
    n = _sz(0)
    _check(lib().ttt_hybrid_block_workspace_size(ctypes.byref(cfg), seg_len, ctypes.byref(n)))
    return n.value


def hybrid_block(cfg: Config, seg_len: int, X, theta_attn, theta_out, theta, W1_0, W2_0, alpha_f, alpha_b, *,
                 workspace=None, out=None):
    """ttt_hybrid_block: returns Y [B, T, D] bf16."""
    import torch
    Y = torch.empty_like(X) if out is None else out
    ws = (torch.empty(max(hybrid_workspace_size(cfg, seg_len), 1), dtype=torch.uint8, device=X.device)
          if workspace is None else workspace)
    _check(lib().ttt_hybrid_block(ctypes.byref(cfg), seg_len, _ptr(X), _ptr(theta_attn), _ptr(theta_out), _ptr(theta),
                                  _ptr(W1_0), _ptr(W2_0), _ptr(alpha_f), _ptr(alpha_b), _ptr(Y), _ptr(ws), ws.numel(),
                                  _stream(X.device)))
    return Y


def project(cfg: Config, X, theta):
    """ttt_mlp_project: QKV [3, B, H, T, d] fp32."""
    import torch
    out = torch.empty((3, cfg.B, cfg.H, cfg.T, cfg.d), dtype=torch.float32, device=X.device)
    _check(lib().ttt_mlp_project(ctypes.byref(cfg), _ptr(X), _ptr(theta), _ptr(out), _stream(X.device)))
    return out


def set_kernel_timing(enable: bool):
    _check(lib().ttt_mlp_set_kernel_timing(int(enable)))


def kernel_timing(kind: int):
    ms, n = ctypes.c_double(0), ctypes.c_int64(0)
    _check(lib().ttt_mlp_kernel_timing(kind, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def reset_kernel_timing():
    _check(lib().ttt_mlp_reset_kernel_timing())
