"""Shared helpers of the GPU tests: moving seeded inputs to the device and
comparing the library's outputs with the oracle's."""
import os

import numpy as np

from test_rnn_layer_amd import workloads as W


def workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def to_device(a, io_dtype, device="cuda"):
    import torch
    if io_dtype == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def from_device(t):
    """Exact float64 copy of a device tensor (bf16 or fp32)."""
    import torch
    if t.dtype == torch.bfloat16:
        bits = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
        return W.bf16_bits_to_f32(bits).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def rel_l2(x, ref):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def max_abs(x, ref):
    return float(np.max(np.abs(np.asarray(x, np.float64) - np.asarray(ref, np.float64)))) if np.size(ref) else 0.0


def rel_l2_tenths(x, ref, axis=1):
    """Relative L2 per tenth of the sequence axis (late tokens are small)."""
    T = np.shape(ref)[axis]
    out = []
    for i in range(10):
        a, b = i * T // 10, (i + 1) * T // 10
        if b > a:
            out.append(rel_l2(np.take(x, range(a, b), axis=axis), np.take(ref, range(a, b), axis=axis)))
    return out


def device_inputs(wl, inp):
    import torch
    return dict(
        X=to_device(inp["X"], wl.io_dtype), theta=to_device(inp["theta"], wl.io_dtype),
        W1_0=torch.from_numpy(inp["W1_0"]).cuda(), W2_0=torch.from_numpy(inp["W2_0"]).cuda(),
        alpha_f=torch.from_numpy(inp["alpha_f"]).cuda(), alpha_b=torch.from_numpy(inp["alpha_b"]).cuda())


def f64_inputs(wl, inp):
    return dict(X=W.to_f64(inp["X"], wl.io_dtype), theta=W.to_f64(inp["theta"], wl.io_dtype),
                W1_0=inp["W1_0"].astype(np.float64), W2_0=inp["W2_0"].astype(np.float64),
                alpha_f=inp["alpha_f"].astype(np.float64), alpha_b=inp["alpha_b"].astype(np.float64))


def host_f32(t, cols=None):
    """float32 host copy of a device tensor [B, T, D] (bf16 widened exactly),
    optionally only the channel columns `cols`."""
    import torch
    if cols is not None:
        t = t[..., torch.as_tensor(cols, device=t.device)]
    if t.dtype == torch.bfloat16:
        return W.bf16_bits_to_f32(t.detach().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().cpu().numpy().astype(np.float32, copy=False)


def head_cols(heads, d):
    """Channel indices of the listed heads, in that order."""
    return np.concatenate([np.arange(h * d, (h + 1) * d) for h in heads]) if len(heads) else np.zeros(0, int)


class TenthsError:
    """Relative L2 error over the whole sequence and per tenth of it, accumulated
    over several pieces of the channel axis (sums of squares in float64)."""

    def __init__(self, T):
        self.T = T
        self.bounds = [(i * T // 10, (i + 1) * T // 10) for i in range(10)]
        self.num = np.zeros(10)
        self.den = np.zeros(10)

    def add(self, got, ref):
        """got, ref: [B, T, n] (or [T, n]) pieces of the same columns."""
        got = np.asarray(got)
        ref = np.asarray(ref)
        if ref.ndim == 2:
            got, ref = got[None], ref[None]
        for i, (a, b) in enumerate(self.bounds):
            r = ref[:, a:b].astype(np.float64)
            e = got[:, a:b].astype(np.float64) - r
            self.num[i] += float(np.sum(e * e))
            self.den[i] += float(np.sum(r * r))

    def overall(self):
        return float(np.sqrt(self.num.sum() / max(self.den.sum(), 1e-300)))

    def tenths(self):
        return [float(np.sqrt(n / max(d, 1e-300))) for n, d in zip(self.num, self.den)]
