"""Benchmark of the TTT-MLP bidirectional layer (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload bidir307k] [--backward]

A step is one ttt_mlp_bidir call over the whole sequence: projections, the
forward scan with its gate, the projections of X', the reversed scan with its
gate.  With --backward a step is one ttt_mlp_bidir_backward call instead (the
gradients of sum(dY * Y) for a seeded dY).  Inputs are seeded synthetic
tensors already resident in device memory.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TTT-MLP bidirectional layer tokens/sec at 307,200 tokens; % of roofline"
METRIC_LINEAR = "TTT-Linear bidirectional layer tokens/sec at 307,200 tokens; % of roofline"
METRIC_BACKWARD = "TTT-MLP bidirectional layer backward tokens/sec at 307,200 tokens; % of roofline"
METRIC_HYBRID = ("Hybrid block (segment-local attention, then the TTT-MLP bidirectional layer) tokens/sec at "
                 "307,200 tokens; % of roofline")


def metric_for(metric: str, wl) -> str:
    """The metric's name with the workload's own token count (B T) in place of 307,200."""
    n = wl.B * wl.T
    return metric if n == 307_200 else metric.replace("307,200", f"{n:,}")
# MI355X published peaks
PEAK_BF16_TFLOPS = 2516.6
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_traffic.json")


def scan_flops_per_token_head(d: int, m: int, b: int) -> int:
    """Algorithmic flops of one scan step per token and head (multiply-add = 2):
    seven d x m contractions (K W1, Hk W2, G2 W2^T, Q W1, Hq W2, K^T G1, Hk^T G2)
    plus the causal halves of the b x b products (tril(QK^T), its product with
    G1, tril(Hq Hk^T), its product with G2)."""
    return 7 * 2 * d * m + (b + 1) * (2 * d + 2 * m)


def linear_scan_flops_per_token_head(d: int, b: int) -> int:
    """The linear inner model: three d x d contractions (K W, Q W, K^T G) plus the
    causal halves of tril(Q K^T) and of its product with G."""
    return 3 * 2 * d * d + (b + 1) * 2 * d


def backward_scan_flops_per_token_head(d: int, m: int, b: int) -> int:
    """Algorithmic flops of the backward scan per token and head: the mini-batch's
    forward quantities again (K W1, Hk W2, G2 W2^T, Q W1: 4 d x m contractions), the
    gradient contractions (dZ W2^T, dAq W1^T, G2 dW2^T, Hk dW2, K dW1, G1 dW1^T, dGh W2,
    dYh W2^T, dA W1^T: 9) and the state adjoints (Q^T dAq, K^T dA, Hq^T dZ, dGh^T G2,
    Hk^T dYh: 5), plus the causal halves of the b x b products (5 over d, 6 over m).
    The replay of each segment from its checkpoint (10 d m per token) is
    recomputation and not counted."""
    return 18 * 2 * d * m + (b + 1) * (5 * d + 6 * m)


def proj_flops_per_token(D: int) -> int:
    return 2 * 3 * D * D


def kernel_digest(kernel: str) -> str:
    from test_rnn_layer_amd.profile_counters import KERNEL_SOURCES, source_digest
    return source_digest(KERNEL_SOURCES[kernel])


def traffic_from_profile(kernel: str, digest: str):
    """HBM bytes per scan launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = rec.get(kernel)
    if not e or e.get("source_digest") != digest:
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(wl, tokens: int):
    """The fp64 oracle on the first `tokens` tokens of the same workload (both
    directions, every head), timed on this host's cores."""
    import numpy as np

    from oracle import ttt_linear_oracle as LO
    from oracle import ttt_oracle as O
    from test_rnn_layer_amd import workloads as W

    sub = wl.replace(T=tokens)
    inp = W.make_inputs(sub)
    X = W.to_f64(inp["X"], sub.io_dtype)
    th = W.to_f64(inp["theta"], sub.io_dtype)
    nw = O.default_workers()
    t0 = time.perf_counter()
    if sub.model == "linear":
        LO.ttt_linear_bidir(X, th, inp["W1_0"].astype(np.float64), inp["alpha_f"].astype(np.float64),
                            inp["alpha_b"].astype(np.float64), eta=sub.eta, b=sub.b, loss=sub.loss, workers=nw)
    else:
        O.ttt_bidir(X, th, inp["W1_0"].astype(np.float64), inp["W2_0"].astype(np.float64),
                    inp["alpha_f"].astype(np.float64), inp["alpha_b"].astype(np.float64),
                    eta=sub.eta, b=sub.b, loss=sub.loss, gelu_form=sub.gelu, workers=nw)
    dt = time.perf_counter() - t0
    return dict(value=tokens / dt, unit="tokens/s", cores=nw, kind="oracle",
                sample=f"{wl.name} workload, first {tokens} of {wl.T} tokens per sequence "
                       f"({100.0 * tokens / wl.T:.1f}% of it), all {wl.H} heads, both directions, fp64 NumPy, "
                       f"{dt:.1f} s wall")


def cpu_baseline_backward(wl, tokens: int):
    """The fp64 backward oracle (autograd through the primal-form layer) on the
    first `tokens` tokens of the same workload, every head, both directions."""
    import numpy as np
    import torch

    from oracle import ttt_backward_oracle as BO
    from test_rnn_layer_amd import workloads as W

    sub = wl.replace(T=tokens)
    inp = W.make_inputs(sub)
    X = W.to_f64(inp["X"], sub.io_dtype)
    th = W.to_f64(inp["theta"], sub.io_dtype)
    dy = W.make_dy(sub).astype(np.float64)
    t0 = time.perf_counter()
    BO.ttt_mlp_bidir_backward(X, th, inp["W1_0"].astype(np.float64), inp["W2_0"].astype(np.float64),
                              inp["alpha_f"].astype(np.float64), inp["alpha_b"].astype(np.float64), dy,
                              eta=sub.eta, b=sub.b, loss=sub.loss, gelu_form=sub.gelu)
    dt = time.perf_counter() - t0
    return dict(value=tokens / dt, unit="tokens/s", cores=torch.get_num_threads(), kind="oracle",
                sample=f"{wl.name} workload, first {tokens} of {wl.T} tokens per sequence "
                       f"({100.0 * tokens / wl.T:.3f}% of it), all {wl.H} heads, both directions, fp64 torch "
                       f"autograd, {dt:.1f} s wall")


def bench_backward(args, wl):
    """--backward: one ttt_mlp_bidir_backward call per step."""
    import numpy as np
    import torch

    from test_rnn_layer_amd import _lib
    from test_rnn_layer_amd import workloads as W

    dev = torch.device("cuda:0")
    inp = W.make_inputs(wl)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    io = bf if wl.io_dtype == "bf16" else f32
    X, th = io(inp["X"]), io(inp["theta"])
    W1, W2 = f32(inp["W1_0"]), f32(inp["W2_0"])
    af, ab = f32(inp["alpha_f"]), f32(inp["alpha_b"])
    dY = f32(W.make_dy(wl))
    del inp
    cfg = _lib.make_config(wl.B, wl.T, wl.H, wl.d, wl.m, wl.b, wl.eta, io_dtype=wl.io_dtype, loss=wl.loss,
                           gelu=wl.gelu)
    ws = torch.empty(_lib.backward_workspace_size(cfg, True), dtype=torch.uint8, device=dev)
    step = lambda: _lib.bidir_backward(cfg, X, th, W1, W2, af, ab, dY, workspace=ws)
    print(f"# bench: backward, inputs resident ({ws.numel() / 1e9:.1f} GB workspace), warming up", file=sys.stderr,
          flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    _lib.set_kernel_timing(True)
    _lib.reset_kernel_timing()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
        torch.cuda.synchronize()
        print(f"# bench: backward step {i + 1} done", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kinds = {"backward_scan": _lib.TTT_KERNEL_BACKWARD, "forward_scan": _lib.TTT_KERNEL_SCAN,
             "projection": _lib.TTT_KERNEL_PROJECT, "gradient_gemms": _lib.TTT_KERNEL_GRAD_GEMM}
    km = {k: _lib.kernel_timing(v) for k, v in kinds.items()}
    _lib.set_kernel_timing(False)
    ms_per_step = elapsed * 1e3 / args.steps
    tokens = wl.B * wl.T
    dirs = 2
    bms, bn = km["backward_scan"]
    fpt = backward_scan_flops_per_token_head(wl.d, wl.m, wl.b)
    flops_launch = fpt * wl.H * tokens * dirs * args.steps / bn
    avg_ms = bms / bn
    achieved = flops_launch / (avg_ms / 1e3) / 1e12
    # layer: the gradient GEMMs (dX and dtheta, 12 D^2 per token and direction) at the bf16 peak,
    # both scans (the forward pass again, and the backward) at the fp32 peak
    gemm_total = 12 * wl.D * wl.D * tokens * dirs
    scan_total = (fpt + scan_flops_per_token_head(wl.d, wl.m, wl.b)) * wl.H * tokens * dirs
    R_ms = (gemm_total / (PEAK_BF16_TFLOPS * 1e12) + scan_total / (PEAK_FP32_TFLOPS * 1e12)) * 1e3
    out = {
        "metric": metric_for(METRIC_BACKWARD, wl), "value": tokens / (ms_per_step / 1e3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "H": wl.H, "d": wl.d, "m": wl.m, "b": wl.b,
                   "eta": wl.eta, "D": wl.D, "directions": dirs, "pass": "backward",
                   "scan_kernel": "scan_backward", "model": wl.model},
        "roofline": {"bound": "alu", "kernel": "scan_backward", "achieved": achieved, "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_TFLOPS, "traffic": None,
                     "flops_per_launch": flops_launch, "avg_launch_ms": avg_ms},
        "layer_roofline": {"R_ms": R_ms, "frac": R_ms / ms_per_step,
                           "definition": "gradient GEMM flops at bf16 MFMA peak + forward and backward scan flops "
                                         "at fp32 peak"},
        "kernel_ms_per_step": {k: ms / args.steps for k, (ms, n) in km.items()},
    }
    if not args.no_cpu_baseline:
        print("# bench: timing the CPU backward oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_backward(wl, args.cpu_tokens or 16)
    print(json.dumps(out), flush=True)


def attention_flops(T: int, L: int, H: int, d: int) -> int:
    """Q K^T and P V over every segment of one sequence (all pairs within a segment)."""
    full, rest = divmod(T, L)
    return 4 * d * H * (full * L * L + rest * rest)


def cpu_baseline_hybrid(wl, tokens: int):
    """The fp64 oracle's hybrid block on the first `tokens` tokens (one segment:
    attention over those tokens, then the bidirectional TTT layer), every head."""
    import numpy as np

    from oracle import attention_oracle as AO
    from oracle import ttt_oracle as O
    from test_rnn_layer_amd import workloads as W

    sub = wl.replace(T=tokens)
    inp = W.make_inputs(sub)
    thA, thO = W.make_attention_weights(sub)
    X = W.to_f64(inp["X"], sub.io_dtype)
    nw = O.default_workers()
    t0 = time.perf_counter()
    AO.hybrid_block(X, W.to_f64(thA, sub.io_dtype), W.to_f64(thO, sub.io_dtype), wl.attn_seg,
                    W.to_f64(inp["theta"], sub.io_dtype), inp["W1_0"].astype(np.float64),
                    inp["W2_0"].astype(np.float64), inp["alpha_f"].astype(np.float64),
                    inp["alpha_b"].astype(np.float64), eta=sub.eta, b=sub.b, loss=sub.loss, gelu_form=sub.gelu,
                    workers=nw)
    dt = time.perf_counter() - t0
    return dict(value=tokens / dt, unit="tokens/s", cores=nw, kind="oracle",
                sample=f"{wl.name} workload, first {tokens} of {wl.T} tokens per sequence "
                       f"({100.0 * tokens / wl.T:.1f}% of it, within one attention segment), all {wl.H} heads, "
                       f"attention and both TTT directions, fp64 NumPy, {dt:.1f} s wall")


def bench_hybrid(args, wl):
    """A step is one ttt_hybrid_block call: the attention projections, the segment
    attention, the output projection with the residual, and the bidirectional TTT layer."""
    import numpy as np
    import torch

    from test_rnn_layer_amd import _lib
    from test_rnn_layer_amd import workloads as W

    dev = torch.device("cuda:0")
    inp = W.make_inputs(wl)
    thA, thO = W.make_attention_weights(wl)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    X, th, tA, tO = bf(inp["X"]), bf(inp["theta"]), bf(thA), bf(thO)
    W1, W2 = f32(inp["W1_0"]), f32(inp["W2_0"])
    af, ab = f32(inp["alpha_f"]), f32(inp["alpha_b"])
    del inp, thA, thO
    cfg = _lib.make_config(wl.B, wl.T, wl.H, wl.d, wl.m, wl.b, wl.eta, io_dtype=wl.io_dtype, loss=wl.loss,
                           gelu=wl.gelu, algo=args.algo)
    ws = torch.empty(_lib.hybrid_workspace_size(cfg, wl.attn_seg), dtype=torch.uint8, device=dev)
    Y = torch.empty_like(X)
    step = lambda: _lib.hybrid_block(cfg, wl.attn_seg, X, tA, tO, th, W1, W2, af, ab, workspace=ws, out=Y)
    print("# bench: hybrid block, inputs resident, warming up", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    _lib.set_kernel_timing(True)
    _lib.reset_kernel_timing()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kinds = {"attention": _lib.TTT_KERNEL_ATTENTION, "scan": _lib.TTT_KERNEL_SCAN, "projection": _lib.TTT_KERNEL_PROJECT}
    km = {k: _lib.kernel_timing(v) for k, v in kinds.items()}
    _lib.set_kernel_timing(False)
    ms_per_step = elapsed * 1e3 / args.steps
    tokens = wl.B * wl.T
    ams, an = km["attention"]
    af_launch = attention_flops(wl.T, wl.attn_seg, wl.H, wl.d) * wl.B
    avg_ms = ams / an
    achieved = af_launch / (avg_ms / 1e3) / 1e12
    # block roofline: attention, the attention projections (Q|K|V and output: 8 D^2 per token) and the TTT
    # projections at the bf16 peak, the TTT scan at the fp32 peak
    mm_total = af_launch + (8 * wl.D * wl.D + proj_flops_per_token(wl.D) * 2) * tokens
    scan_total = scan_flops_per_token_head(wl.d, wl.m, wl.b) * wl.H * tokens * 2
    R_ms = (mm_total / (PEAK_BF16_TFLOPS * 1e12) + scan_total / (PEAK_FP32_TFLOPS * 1e12)) * 1e3
    out = {
        "metric": metric_for(METRIC_HYBRID, wl), "value": tokens / (ms_per_step / 1e3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "H": wl.H, "d": wl.d, "m": wl.m, "b": wl.b,
                   "eta": wl.eta, "D": wl.D, "attention_segment": wl.attn_seg, "directions": 2,
                   "scan_kernel": "scan_" + _lib.select_algo(cfg), "model": wl.model},
        "roofline": {"bound": "mfma", "kernel": "segment_attention", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "flops_per_launch": af_launch, "avg_launch_ms": avg_ms},
        "layer_roofline": {"R_ms": R_ms, "frac": R_ms / ms_per_step,
                           "definition": "attention and projection flops at bf16 MFMA peak + TTT scan flops at "
                                         "fp32 peak"},
        "kernel_ms_per_step": {k: ms / args.steps for k, (ms, n) in km.items()},
    }
    if not args.no_cpu_baseline:
        print("# bench: timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_hybrid(wl, args.cpu_tokens or 4096)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="bidir307k")
    ap.add_argument("--algo", default="auto", choices=["auto", "generic", "mfma"])
    ap.add_argument("--cpu-tokens", type=int, default=None,
                    help="tokens of the CPU oracle's sample (default 24576; 16 with --backward, 4096 for the "
                         "hybrid block)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true", help="time ttt_mlp_bidir_backward instead")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the layer's heads would shard across GPUs, and this program "
              f"times the one GPU's share only; --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from test_rnn_layer_amd import _lib
    from test_rnn_layer_amd import workloads as W

    wl = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"# bench: workload {wl.name} B={wl.B} T={wl.T} H={wl.H} d={wl.d} m={wl.m} b={wl.b}", file=sys.stderr,
          flush=True)
    if args.backward:
        if wl.model != "mlp":
            print("bench.py --backward: the backward covers the MLP model only", file=sys.stderr)
            sys.exit(2)
        return bench_backward(args, wl)
    if wl.attn_seg > 0:
        return bench_hybrid(args, wl)
    inp = W.make_inputs(wl)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    io = bf if wl.io_dtype == "bf16" else f32
    X, th = io(inp["X"]), io(inp["theta"])
    W1, W2 = f32(inp["W1_0"]), f32(inp["W2_0"])
    af, ab = f32(inp["alpha_f"]), f32(inp["alpha_b"])
    del inp
    linear = wl.model == "linear"
    cfg = _lib.make_config(wl.B, wl.T, wl.H, wl.d, wl.m, wl.b, wl.eta, io_dtype=wl.io_dtype, loss=wl.loss,
                           gelu=wl.gelu, algo=args.algo, model=wl.model)
    if linear:
        W2 = None  # the linear model has one d x d state
    ws = torch.empty(_lib.workspace_size(cfg, True), dtype=torch.uint8, device=dev)
    Y = torch.empty_like(X)
    step = lambda: _lib.bidir(cfg, X, th, W1, W2, af, ab, workspace=ws, out=Y)
    print("# bench: inputs resident, warming up", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    _lib.set_kernel_timing(True)
    _lib.reset_kernel_timing()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    scan_ms, scan_n = _lib.kernel_timing(_lib.TTT_KERNEL_SCAN)
    proj_ms, proj_n = _lib.kernel_timing(_lib.TTT_KERNEL_PROJECT)
    _lib.set_kernel_timing(False)
    print(f"# bench: {args.steps} steps in {elapsed:.3f} s; scan {scan_n} launches {scan_ms:.1f} ms; "
          f"projection {proj_n} launches {proj_ms:.1f} ms", file=sys.stderr, flush=True)

    ms_per_step = elapsed * 1e3 / args.steps
    tokens = wl.B * wl.T
    value = tokens / (ms_per_step / 1e3)
    dirs = 2
    # dominant kernel: the scan; one launch covers one direction of the whole batch
    scan_fpt = linear_scan_flops_per_token_head(wl.d, wl.b) if linear else scan_flops_per_token_head(wl.d, wl.m, wl.b)
    scan_flops_launch = scan_fpt * wl.H * tokens * dirs * args.steps / scan_n
    scan_avg_ms = scan_ms / scan_n
    achieved = scan_flops_launch / (scan_avg_ms / 1e3) / 1e12
    algo = _lib.select_algo(cfg)
    used_mfma = algo == "mfma"
    peak = PEAK_BF16_TFLOPS if used_mfma else PEAK_FP32_TFLOPS
    kname = ("scan_linear_" if linear else "scan_") + algo
    traffic = traffic_from_profile(kname, kernel_digest(kname))
    # layer roofline: projections at bf16 MFMA peak plus the scan at fp32 peak
    proj_total = proj_flops_per_token(wl.D) * tokens * dirs
    scan_total = scan_fpt * wl.H * tokens * dirs
    R_ms = (proj_total / (PEAK_BF16_TFLOPS * 1e12) + scan_total / (PEAK_FP32_TFLOPS * 1e12)) * 1e3
    # the same with the scan's contractions priced at the bf16 peak (they run on bf16 operands)
    R_exec_ms = (proj_total + scan_total) / (PEAK_BF16_TFLOPS * 1e12) * 1e3
    out = {
        "metric": metric_for(METRIC_LINEAR if linear else METRIC, wl), "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "H": wl.H, "d": wl.d, "m": wl.m, "b": wl.b,
                   "eta": wl.eta, "D": wl.D, "directions": dirs, "scan_kernel": kname, "model": wl.model},
        "roofline": {"bound": "mfma" if used_mfma else "alu", "kernel": kname, "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "flops_per_launch": scan_flops_launch, "avg_launch_ms": scan_avg_ms},
        "layer_roofline": {"R_ms": R_ms, "frac": R_ms / ms_per_step,
                           "definition": "projection flops at bf16 MFMA peak + scan flops at fp32 peak"},
        "kernel_ms_per_step": {"scan": scan_ms / args.steps, "projection": proj_ms / args.steps},
    }
    if used_mfma:  # the scan's contractions run on bf16 operands: the same sum with them at the bf16 peak
        out["layer_roofline"].update(R_exec_ms=R_exec_ms, frac_exec=R_exec_ms / ms_per_step)
    if not args.no_cpu_baseline:
        print("# bench: timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_tokens or 24576)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
