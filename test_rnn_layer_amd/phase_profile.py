"""Per-phase cycle breakdown of a scan step, from the phase-marks build.

    python -m test_rnn_layer_amd.build --phase-marks
    python -m test_rnn_layer_amd.phase_profile --kernel mfma [--workload bidir307k] [--tokens N] [--out FILE]

Runs one direction of the layer (ttt_mlp_forward; with --kernel backward its
backward, ttt_mlp_backward, whose backward scan is marked per mini-batch) on the
measurement build libttt_mlp_marks.so, whose scan kernels store the shader clock
at the phase boundaries of kMarkSteps steps of workgroup 0, wave 0 (see
csrc/phase_marks.h), and prints the median cycles of each phase and of a whole
step.  The marks add
a wait for each clock read, so the marked step is somewhat longer than the
library's; the clock is estimated from the marked step's cycles and the
launch times of the same run (HIP events).
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MARK_STEPS, MARK_PHASES = 256, 8  # csrc/phase_marks.h: kMarkSteps, kMarkPhases

PHASES = {
    "mfma": [
        "state to bf16; A = K W1, S = K Q^T; GELU(A); partial Yhat = Hk W2 -> LDS",
        "first barrier",
        "Yhat summed over the waves; -eta G2 -> LDS",
        "Z of block j-2 summed over the waves",
        "GELU'(A) -> LDS; transposed operands read back; wait for vector memory",
        "second barrier",
        "Gh, G1; W1, W2, W2^T updates; read-out of block j-1 (Aq, GELU(Aq), causal products, partial Z -> LDS); gate and stores of block j-2; staging",
        "loop to the next step",
    ],
    "coop": [
        "loads of v_t and the next k, q (no barrier: the partials of a are complete since the last gather)",
        "GELU(a), GELU(aq); first W2 pass (partial yhat, z); barrier",
        "publish this workgroup's partials (device-scope stores)",
        "the previous token's W1 update and the next pre-activations; poll the other workgroups' partials",
        "barrier after the gather",
        "sums, gate store; G2; W2 update; G2 W2^T reduction; barrier (and the stop flag of a failed poll)",
        "G1 of this token (its W1 update follows in the next token's exchange)",
        "loop to the next token",
    ],
    "backward": [  # the walk split over several workgroups per chain (bidir307k's shape: four)
        "barrier; the state part, K/Q rows, G2, M and the seven panels into LDS, dZ = tanh(alpha) dY; barrier",
        "N (this part), dN, dZ W2^T; barrier",
        "dHq = dZ W2^T + dN Hk (dAq in its epilogue), dN^T Hq, N^T dZ; barrier",
        "dQ, dM (this part), the products with the adjoint part; dG1 = -eta (K dW1' + M^T dAq) (dGh, dA in its epilogue); barrier",
        "dQ += dM K (dQ out from its epilogue), dK += dM^T Q, dG2 += dGh W2; barrier",
        "dG2's partials exchanged with the other parts (publish, poll); barrier",
        "dHk += dYh W2^T (dA += dHk S1 in its epilogue); barrier; dK += dA W1^T (dK out from its epilogue)",
        "dV stores, the rank-16 updates of the adjoint part; loop",
    ],
}
ENTRY = {"mfma": "ttt_phase_marks_scan_mfma", "coop": "ttt_phase_marks_scan_coop",
         "backward": "ttt_phase_marks_scan_backward"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--kernel", choices=list(PHASES), default="mfma")
    ap.add_argument("--workload", default=None, help="default: bidir307k (mfma), bigstate307k (coop)")
    ap.add_argument("--tokens", type=int, default=None, help="tokens of the sequence (default: the workload's)")
    ap.add_argument("--reverse", action="store_true")
    ap.add_argument("--out", default=None, help="also write the table (markdown) to this file")
    args = ap.parse_args()

    import torch

    from test_rnn_layer_amd import _lib, build
    from test_rnn_layer_amd import workloads as W

    if not os.path.exists(build.MARKS_LIB_PATH):
        raise SystemExit(f"{build.MARKS_LIB_PATH} is missing: python -m test_rnn_layer_amd.build --phase-marks")
    _lib.use_library(build.MARKS_LIB_PATH)
    L = _lib.lib()
    fn = getattr(L, ENTRY[args.kernel])
    fn.restype = ctypes.c_int32
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64]

    name = args.workload or ("bigstate307k" if args.kernel == "coop" else "bidir307k")
    wl = W.WORKLOADS[name]
    if args.tokens:
        wl = wl.replace(T=args.tokens)
    dev = torch.device("cuda:0")
    inp = W.make_inputs(wl)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    X, th = bf(inp["X"]), bf(inp["theta"])
    W1, W2, al = f32(inp["W1_0"]), f32(inp["W2_0"]), f32(inp["alpha_f"])
    bwd = args.kernel == "backward"
    cfg = _lib.make_config(wl.B, wl.T, wl.H, wl.d, wl.m, wl.b, wl.eta, io_dtype=wl.io_dtype,
                           algo="auto" if bwd else args.kernel)
    print(f"# phase marks: {args.kernel} scan, {wl.name} B={wl.B} T={wl.T} H={wl.H}, one direction", flush=True)
    if bwd:
        dY = torch.from_numpy(W.make_dy(wl)).to(dev)
        ws = torch.empty(_lib.backward_workspace_size(cfg, False), dtype=torch.uint8, device=dev)
        run = lambda: _lib.backward(cfg, X, th, W1, W2, al, dY, reverse=args.reverse, workspace=ws)
    else:
        ws = torch.empty(_lib.workspace_size(cfg, False), dtype=torch.uint8, device=dev)
        run = lambda: _lib.forward(cfg, X, th, W1, W2, al, reverse=args.reverse, workspace=ws)
    run()
    torch.cuda.synchronize()
    _lib.set_kernel_timing(True)
    _lib.reset_kernel_timing()
    run()
    torch.cuda.synchronize()
    scan_ms, scan_n = _lib.kernel_timing(_lib.TTT_KERNEL_BACKWARD if bwd else _lib.TTT_KERNEL_SCAN)
    _lib.set_kernel_timing(False)
    marks = np.zeros(MARK_STEPS * MARK_PHASES, dtype=np.uint64)
    assert fn(marks.ctypes.data, marks.size) == 0, "reading the marks failed"
    m = marks.reshape(MARK_STEPS, MARK_PHASES).astype(np.int64)
    # the launches of one direction together take every step of the sequence once
    steps = wl.T if args.kernel == "coop" else -(-wl.T // wl.b)
    step_us = scan_ms * 1e3 / steps
    valid = np.all(m > 0, axis=1)
    n = int(np.argmin(valid)) if not valid.all() else MARK_STEPS
    if n < 2:
        raise SystemExit("fewer than two marked steps: the launch was shorter than the marked window")
    m = m[:n]
    d = np.diff(m, axis=1)[:-1]                  # phases 0..6 within a step
    loop = m[1:, 0] - m[:-1, MARK_PHASES - 1]    # phase 7: end of a step to the start of the next
    step = m[1:, 0] - m[:-1, 0]
    # a later, shorter launch overwrites only the first marks of the window: keep the
    # consecutive steps of one launch (every phase and the step itself forward in time)
    ok = np.all(d >= 0, axis=1) & (loop >= 0) & (step > 0)
    d, loop, step = d[ok], loop[ok], step[ok]
    med = [float(np.median(d[:, p])) for p in range(MARK_PHASES - 1)] + [float(np.median(loop))]
    tot = float(np.median(step))
    clock = tot / step_us  # cycles per microsecond (MHz)
    lines = [
        f"Phase breakdown of one {args.kernel} scan step (phase-marks build, workgroup 0 wave 0, "
        f"medians over {int(ok.sum())} steps), {wl.name} T={wl.T} H={wl.H}, "
        f"{'reversed' if args.reverse else 'forward'} direction.",
        "",
        f"Scan kernel time of the direction: {scan_ms:.2f} ms over {scan_n} launches, {step_us:.3f} us per step; "
        f"marked step median {tot:.0f} cycles, i.e. a clock of about {clock:.0f} MHz.",
        "",
        "| # | phase | median cycles | share | us at that clock |",
        "|---|---|---|---|---|",
    ]
    for p, (name_p, c) in enumerate(zip(PHASES[args.kernel], med)):
        lines.append(f"| {p} | {name_p} | {c:.0f} | {100 * c / tot:.1f}% | {c / clock:.3f} |")
    lines.append(f"| | whole step (median of step-to-step) | {tot:.0f} | 100% | {tot / clock:.3f} |")
    text = "\n".join(lines)
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    main()
