"""Seeded synthetic workloads for the TTT-MLP layer scan.

This module only draws inputs.  It holds none of the layer's arithmetic: it
makes the token matrix X, the outer-loop projections theta_Q/theta_K/theta_V,
the initial inner-model state W1_0/W2_0 and the gate vectors alpha, and it
converts between the stored formats (fp32, or bf16 kept as uint16 bit
patterns) and float64.  Both the HIP path (through the Python binding) and
the CPU oracle take their inputs from here; nothing here calls either.

Shapes follow "One-Minute Video Generation with Test-Time Training"
(paper-notes page, section on key designs, "TTT-MLP layer" and "gate +
bidirectional"): tokens are rows of a [B, T, D] matrix with D = H * d, each
head owns a d-wide slice of the channels, its hidden state is a two-layer
MLP with hidden width m = 4d.  The sizes stand in for the video model's
activations (one minute of video is more than 300k tokens, 18 s about 100k,
one 3-s segment 14,400); the video data and the pretrained weights are not
used.

Generator: numpy PCG64 seeded with SeedSequence([seed, tensor_id, chunk]),
normal draws in float64, scaled, cast to float32 and, for bf16 workloads,
rounded to bf16 with round-to-nearest-even.  X is drawn in chunks of
X_CHUNK rows so that any token range can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

# tensor ids inside the seed sequence
TID_X, TID_THETA_Q, TID_THETA_K, TID_THETA_V, TID_W1, TID_W2, TID_SEGMEAN, TID_DY, TID_THETA_A, TID_THETA_O = range(10)
X_CHUNK = 4096


@dataclass(frozen=True)
class Workload:
    """One layer configuration plus the recipe of its synthetic inputs."""

    name: str
    B: int
    T: int
    H: int
    d: int
    m: int
    b: int
    eta: float
    bidir: bool
    io_dtype: str  # "f32" or "bf16"
    alpha_f: float = 0.1
    alpha_b: float = 0.1
    seg_len: int = 0  # 0: no per-segment mean shift
    seg_var: float = 0.0
    seed: int = 0
    loss: str = "mean"  # "mean" (1/d)||e||^2, or "sum" ||e||^2
    gelu: str = "erf"  # "erf" (exact) or "tanh" (approximation)
    model: str = "mlp"  # "mlp": f(u; W) = GELU(u W1) W2; "linear": f(u; W) = u W with W = W1 (m = d)
    attn_seg: int = 0  # > 0: the hybrid block, segment-local attention over segments of this many tokens

    @property
    def D(self) -> int:
        return self.H * self.d

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five layer configurations.  eta for the b=16 layers is 0.1/b.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", B=1, T=256, H=1, d=16, m=64, b=1, eta=0.1,
                         bidir=False, io_dtype="f32"),
    "seg14k": Workload("seg14k", B=1, T=14_400, H=48, d=64, m=256, b=16, eta=0.1 / 16,
                       bidir=False, io_dtype="bf16"),
    "bidir100k": Workload("bidir100k", B=1, T=100_800, H=48, d=64, m=256, b=16,
                          eta=0.1 / 16, bidir=True, io_dtype="bf16"),
    "bidir307k": Workload("bidir307k", B=1, T=307_200, H=48, d=64, m=256, b=16,
                          eta=0.1 / 16, bidir=True, io_dtype="bf16",
                          seg_len=14_400, seg_var=0.25),
    "bigstate307k": Workload("bigstate307k", B=1, T=307_200, H=24, d=128, m=512, b=1,
                             eta=0.05, bidir=True, io_dtype="bf16"),
}
WORKLOAD_ORDER = ["tiny_f32", "seg14k", "bidir100k", "bidir307k", "bigstate307k"]
# TTT-Linear (the same layer with a linear inner model, d x d state) at the shape of bidir307k
WORKLOADS["linear307k"] = WORKLOADS["bidir307k"].replace(name="linear307k", m=64, model="linear")
# the hybrid block (segment-local attention over 3-second segments of 14,400 tokens, then the
# bidirectional TTT-MLP layer) at the shape of bidir307k
WORKLOADS["hybrid307k"] = WORKLOADS["bidir307k"].replace(name="hybrid307k", attn_seg=14_400)
# the same 307,200 tokens as 2 or 4 sequences: the scan then runs on 96 or 192 CUs
WORKLOADS["batch2x153k"] = WORKLOADS["bidir307k"].replace(name="batch2x153k", B=2, T=153_600)
WORKLOADS["batch4x76k"] = WORKLOADS["bidir307k"].replace(name="batch4x76k", B=4, T=76_800)


# ----------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> 16) & 1
    lsb += 0x7FFF
    lsb += u  # no wrap-around: finite values stay below 0xFF800000
    lsb >>= 16
    return lsb.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f64(a: np.ndarray, io_dtype: str) -> np.ndarray:
    """Exact widening of a stored input (fp32 or bf16 bits) to float64."""
    if io_dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _store(a64: np.ndarray, io_dtype: str) -> np.ndarray:
    a32 = a64.astype(np.float32)
    return f32_to_bf16_bits(a32) if io_dtype == "bf16" else a32


def _rng(seed: int, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *ids])))


# ----------------------------------------------------------------------------
# tensors
# ----------------------------------------------------------------------------

def segment_means(wl: Workload) -> np.ndarray:
    """Per-segment mean vectors mu_s ~ N(0, seg_var * I_D), float64 [n_seg, D]."""
    n_seg = -(-wl.T // wl.seg_len)
    g = _rng(wl.seed, TID_SEGMEAN)
    return g.standard_normal((n_seg, wl.D)) * np.sqrt(wl.seg_var)


def make_x(wl: Workload, t0: int = 0, t1: int | None = None, seq: int | None = None) -> np.ndarray:
    """Tokens [B, t1-t0, D] (or [t1-t0, D] for one sequence), stored format.

    x_t ~ N(0, I), plus the mean of the token's segment when seg_len > 0.
    Rows t0..t1 are identical to the same rows of the whole sequence.
    """
    t1 = wl.T if t1 is None else t1
    assert 0 <= t0 <= t1 <= wl.T
    seqs = range(wl.B) if seq is None else [seq]
    out = np.empty((len(seqs), t1 - t0, wl.D),
                   dtype=np.uint16 if wl.io_dtype == "bf16" else np.float32)
    mu = segment_means(wl) if wl.seg_len > 0 else None
    def fill(job):
        si, s, c = job
        r0, r1 = c * X_CHUNK, min((c + 1) * X_CHUNK, wl.T)
        a, z = max(r0, t0), min(r1, t1)
        chunk = _rng(wl.seed, TID_X, s, c).standard_normal((r1 - r0, wl.D))[a - r0:z - r0]
        if mu is not None:
            chunk += mu[np.arange(a, z) // wl.seg_len]
        out[si, a - t0:z - t0] = _store(chunk, wl.io_dtype)

    jobs = [(si, s, c) for si, s in enumerate(seqs) for c in range(t0 // X_CHUNK, -(-t1 // X_CHUNK))]
    if len(jobs) > 1:
        with ThreadPoolExecutor(max_workers=min(16, len(jobs))) as ex:
            list(ex.map(fill, jobs))
    else:
        for j in jobs:
            fill(j)
    return out if seq is None else out[0]


def make_theta(wl: Workload) -> np.ndarray:
    """theta_Q, theta_K, theta_V stacked [3, D, D], each [out, in], N(0, 1/D)."""
    D = wl.D
    th = np.empty((3, D, D), dtype=np.uint16 if wl.io_dtype == "bf16" else np.float32)
    for p, tid in enumerate((TID_THETA_Q, TID_THETA_K, TID_THETA_V)):
        th[p] = _store(_rng(wl.seed, tid).standard_normal((D, D)) / np.sqrt(D), wl.io_dtype)
    return th


def make_w0(wl: Workload) -> tuple[np.ndarray, np.ndarray]:
    """Initial state W1_0 [H, d, m] ~ N(0, 1/d) and W2_0 [H, m, d] ~ N(0, 1/m), float32.
    For the linear model (m = d) W1_0 is the state W_0 and W2_0 goes unused."""
    w1 = _rng(wl.seed, TID_W1).standard_normal((wl.H, wl.d, wl.m)) / np.sqrt(wl.d)
    w2 = _rng(wl.seed, TID_W2).standard_normal((wl.H, wl.m, wl.d)) / np.sqrt(wl.m)
    return w1.astype(np.float32), w2.astype(np.float32)


def make_alpha(wl: Workload, value: float | None = None) -> np.ndarray:
    """Gate vector alpha [D], float32 (every channel starts at the same value)."""
    return np.full(wl.D, wl.alpha_f if value is None else value, dtype=np.float32)


def make_dy(wl: Workload, t1: int | None = None, heads=None) -> np.ndarray:
    """An upstream gradient of the layer output, dY [B, T, D] float32 ~ N(0, 1).
    t1 / heads: zero from token t1 on (only the first t1 rows are drawn), and
    outside the listed heads' channels."""
    n = wl.T if t1 is None else t1
    g = np.zeros((wl.B, wl.T, wl.D), dtype=np.float32)
    g[:, :n] = _rng(wl.seed, TID_DY).standard_normal((wl.B, n, wl.D))
    if heads is not None:
        keep = np.zeros(wl.D, dtype=bool)
        for h in heads:
            keep[h * wl.d:(h + 1) * wl.d] = True
        g[..., ~keep] = 0.0
    return g


def make_attention_weights(wl: Workload) -> tuple[np.ndarray, np.ndarray]:
    """The hybrid block's attention projections, stored format: theta_A [3, D, D]
    (Q, K, V, each [out, in]) and theta_O [D, D], every entry N(0, 1/D)."""
    D = wl.D
    thA = _store(_rng(wl.seed, TID_THETA_A).standard_normal((3, D, D)) / np.sqrt(D), wl.io_dtype)
    thO = _store(_rng(wl.seed, TID_THETA_O).standard_normal((D, D)) / np.sqrt(D), wl.io_dtype)
    return thA, thO


def make_inputs(wl: Workload) -> dict:
    """All inputs of one call, in stored format."""
    w1, w2 = make_w0(wl)
    return dict(X=make_x(wl), theta=make_theta(wl), W1_0=w1, W2_0=w2,
                alpha_f=make_alpha(wl, wl.alpha_f), alpha_b=make_alpha(wl, wl.alpha_b))
