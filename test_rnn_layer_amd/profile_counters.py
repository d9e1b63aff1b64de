"""Counters of the scan and projection kernels from rocprofv3 (HBM traffic, and
the shader sequencer's issue, matrix-core and LDS counters).

HBM traffic (one counter per run; each run: a known-size copy, then one layer call):

    rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d DIR_F -o run -- \
        python3 -m test_rnn_layer_amd.profile_counters run
    rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d DIR_W -o run -- \
        python3 -m test_rnn_layer_amd.profile_counters run
    python3 -m test_rnn_layer_amd.profile_counters summarize DIR_F DIR_W

`run` makes one device-to-device copy of COPY_BYTES (the runtime's copy
kernel reads and writes exactly that many bytes), then one ttt_mlp_bidir
call of the workload.  `summarize` scales each counter by what it read for
the copy, writes each kernel's bytes per launch into
profiles/scan_traffic.json, keyed by kernel, with a digest of the kernel's
sources so that a later kernel change invalidates it, and the table
profiles/scan_mfma_proj_tiles_bidir307k_traffic.md.

Sequencer counters (three passes, SQ_PASSES; each fits the per-run limit of
eight SQ counters):

    rocprofv3 --pmc <SQ_PASSES[i]> --kernel-trace --output-format csv -d DIR_i -o run -- \
        python3 -m test_rnn_layer_amd.profile_counters run
    python3 -m test_rnn_layer_amd.profile_counters summarize-sq DIR_1 DIR_2 DIR_3

`summarize-sq` writes profiles/scan_mfma_bidir307k_sq_counters.md: per scan
step, the cycles each unit is busy (vector ALU, matrix core, LDS), LDS bytes
and bank-conflict cycles, waits, and instruction counts.

Kernel times (the bench command under the kernel trace; its JSON line is kept
beside the trace):

    mkdir -p DIR && rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o run -- \
        python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline > DIR/bench.json
    python3 -m test_rnn_layer_amd.profile_counters summarize-stats DIR

`summarize-stats` writes profiles/<scan kernel>_proj_tiles_<workload>_stats.md;
`summarize-backward DIR` (a traced `bench.py --backward` run) writes
profiles/scan_backward_<workload>_stats.md.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 1 << 30
SQ_PASSES = [
    "SQ_WAVES SQ_WAVE_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_SCA SQ_WAIT_INST_ANY "
    "SQ_WAIT_INST_LDS SQ_INSTS_VALU GRBM_GUI_ACTIVE",
    "SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES "
    "SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_INSTS_VALU_MFMA_MOPS_BF16",
    "SQ_INSTS_LDS_LOAD_BANDWIDTH SQ_INSTS_LDS_STORE_BANDWIDTH SQ_INSTS_VALU_TRANS_F32 SQ_WAIT_ANY SQ_BUSY_CU_CYCLES",
]
KERNELS = {"scan_mfma": "scan_mfma_kernel", "scan_generic": "scan_generic_kernel", "scan_coop": "scan_coop_kernel",
           "scan_linear_mfma": "scan_linear_mfma_kernel", "scan_linear_generic": "scan_linear_generic_kernel",
           "projection": "proj_tiles_kernel"}
# the sources each kernel is built from: its counters are stale once any of them changes
KERNEL_SOURCES = {"scan_mfma": ["scan_mfma.hip", "token_block.h", "mfma_common.h", "phi_poly.h", "phase_marks.h",
                                "internal.h"],
                  "scan_generic": ["generic.hip", "internal.h"],
                  "scan_coop": ["scan_coop.hip", "phase_marks.h", "internal.h"],
                  "scan_linear_mfma": ["scan_linear.hip", "token_block.h", "mfma_common.h", "internal.h"],
                  "scan_linear_generic": ["generic.hip", "internal.h"],
                  "scan_backward": ["backward.hip", "internal.h"],
                  "projection": ["proj_mfma.hip", "mfma_common.h", "internal.h"]}


def source_digest(names) -> str:
    h = hashlib.sha256()
    for n in names:
        p = os.path.join(ROOT, "test_rnn_layer_amd", "csrc", n)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def run(workload: str = "bidir307k"):
    import numpy as np
    import torch

    from test_rnn_layer_amd import _lib
    from test_rnn_layer_amd import workloads as W

    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    wl = W.WORKLOADS[workload]
    inp = W.make_inputs(wl)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    io = bf if wl.io_dtype == "bf16" else f32
    cfg = _lib.make_config(wl.B, wl.T, wl.H, wl.d, wl.m, wl.b, wl.eta, io_dtype=wl.io_dtype, loss=wl.loss,
                           gelu=wl.gelu)
    X, th = io(inp["X"]), io(inp["theta"])
    _lib.bidir(cfg, X, th, f32(inp["W1_0"]), f32(inp["W2_0"]), f32(inp["alpha_f"]), f32(inp["alpha_b"]))
    torch.cuda.synchronize()
    print(f"profile_counters: copy of {COPY_BYTES} B and one {workload} bidir call done", flush=True)


def _counter_rows(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def _per_kernel(rows, counter: str):
    """Mean counter value (as reported, KiB) per dispatch of each kernel, and the
    value of the first runtime copy dispatch (the calibration copy: the later
    small copies are the run's host-to-device uploads)."""
    out = {}
    copies = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        name = r.get("Kernel_Name", "")
        disp = int(r.get("Dispatch_Id") or r.get("Correlation_Id"))
        v = float(r["Counter_Value"])
        if "copyBuffer" in name:
            copies[disp] = copies.get(disp, 0.0) + v
            continue
        key = next((k for k, s in KERNELS.items() if s in name), None)
        if key is None:
            continue
        out.setdefault(key, {}).setdefault(disp, 0.0)
        out[key][disp] += v  # a counter may be reported per instance: sum per dispatch
    res = {k: sum(d.values()) / len(d) for k, d in out.items()}
    if copies:
        res["copy"] = copies[min(copies)]
    return res


def summarize(dir_fetch: str, dir_write: str, out_json: str | None = None):
    fetch = _per_kernel(_counter_rows(dir_fetch), "FETCH_SIZE")
    write = _per_kernel(_counter_rows(dir_write), "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("the copy kernel's counters are missing")
    sf = COPY_BYTES / fetch["copy"]  # bytes per counter unit, reads
    sw = COPY_BYTES / write["copy"]  # bytes per counter unit, writes
    rec = {}
    for k in KERNELS:
        if k in fetch and k in write:
            rec[k] = {"bytes_per_launch": fetch[k] * sf + write[k] * sw, "fetch_bytes": fetch[k] * sf,
                      "write_bytes": write[k] * sw, "fetch_counter": fetch[k], "write_counter": write[k],
                      "copy_scale_fetch": sf, "copy_scale_write": sw,
                      "source_digest": source_digest(KERNEL_SOURCES[k])}
    out_json = out_json or os.path.join(ROOT, "profiles", "scan_traffic.json")
    json.dump(rec, open(out_json, "w"), indent=1)
    _traffic_markdown(rec, fetch["copy"], write["copy"], dir_fetch, dir_write)
    print(json.dumps(rec, indent=1))


def _launch_stats(d: str):
    """Per kernel: dispatch count, mean duration (ms) and resource columns, from the
    kernel trace of a counter run."""
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    out = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            key = next((k for k, sub in KERNELS.items() if sub in r.get("Kernel_Name", "")), None)
            if key is None:
                continue
            e = out.setdefault(key, {"n": 0, "ns": 0.0, "row": r})
            e["n"] += 1
            e["ns"] += float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return out


def _traffic_markdown(rec, copy_f, copy_w, dir_f, dir_w):
    from test_rnn_layer_amd import workloads as W
    wl = W.WORKLOADS["bidir307k"]
    launches = _launch_stats(dir_f)
    tok = wl.B * wl.T
    lines = [
        "# HBM traffic per launch, bidir307k (rocprofv3 counters)", "",
        f"Workload: B={wl.B}, T={wl.T:,}, H={wl.H}, d={wl.d}, m={wl.m}, b={wl.b}, bf16 X/θ/Y, fp32 state; "
        "one `ttt_mlp_bidir` call (each direction runs as chunked launches of the projection and the scan).", "",
        "Commands (repo root, MI355X). The copy, of 1 GiB, comes first in each run:", "",
        f"    rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d {dir_f} -o run -- "
        "python3 -m test_rnn_layer_amd.profile_counters run",
        f"    rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d {dir_w} -o run -- "
        "python3 -m test_rnn_layer_amd.profile_counters run",
        f"    python3 -m test_rnn_layer_amd.profile_counters summarize {dir_f} {dir_w}", "",
        f"**Calibration.** The runtime's copy of 1 GiB read FETCH_SIZE = {copy_f:,.1f} and WRITE_SIZE = "
        f"{copy_w:,.1f} (KiB as reported): bytes = FETCH_SIZE × {COPY_BYTES / copy_f:,.1f} and WRITE_SIZE × "
        f"{COPY_BYTES / copy_w:,.1f}.", "",
        "| Kernel | Launches | Read per launch | Written per launch | Whole call (read + written) | Algorithmic, whole call |",
        "|---|---|---|---|---|---|",
    ]
    algo = {"scan_mfma": (2 * tok * wl.D * 2 * 3 + 2 * tok * wl.D * 2 + 2 * tok * wl.D * 2,
                          "token blocks Q, K, V read + gate input read + Y written, both directions"),
            "projection": (2 * (tok * wl.D * 2 + 3 * wl.D * wl.D * 2 + 3 * tok * wl.D * 2),
                           "X read + θ read + token blocks written, both directions")}
    for k, e in rec.items():
        n = launches.get(k, {}).get("n", 0)
        a, what = algo.get(k, (0, ""))
        lines.append(f"| `{KERNELS[k]}` | {n} | {e['fetch_bytes'] / 1e9:.3f} GB | {e['write_bytes'] / 1e9:.3f} GB | "
                     f"{e['bytes_per_launch'] * n / 1e9:.2f} GB | {a / 1e9:.2f} GB ({what}) |")
    lines += ["", "Digests of the sources each row was taken on (profiles/scan_traffic.json): " +
              ", ".join(f"{k} {e['source_digest']}" for k, e in rec.items()) + "."]
    open(os.path.join(ROOT, "profiles", "scan_mfma_proj_tiles_bidir307k_traffic.md"), "w").write(
        "\n".join(lines) + "\n")


def _sq_totals(dirs):
    """Sum of each counter over all dispatches of each kernel, across the pass directories."""
    tot = {}
    for d in dirs:
        for r in _counter_rows(d):
            key = next((k for k, sub in KERNELS.items() if sub in r.get("Kernel_Name", "")), None)
            if key is None:
                continue
            t = tot.setdefault(key, {})
            t[r["Counter_Name"]] = t.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return tot


def summarize_sq(dirs, out_md: str | None = None):
    from test_rnn_layer_amd import workloads as W
    wl = W.WORKLOADS["bidir307k"]
    tot = _sq_totals(dirs)["scan_mfma"]
    launches = _launch_stats(dirs[0])["scan_mfma"]
    row = launches["row"]
    nblk = (wl.T + wl.b - 1) // wl.b
    wg = wl.B * wl.H                      # workgroups (one per sequence and head), 8 waves, 4 SIMDs each
    cu_steps = wg * 2 * nblk              # both directions
    wave_steps = cu_steps * 8
    simd_steps = cu_steps * 4
    q = 4.0                               # quad-cycle counters
    step = tot["SQ_WAVE_CYCLES"] * q / wave_steps      # cycles a wave spends per step
    dur_ns = launches["ns"]
    clock = tot["GRBM_GUI_ACTIVE"] / 8 / dur_ns      # GHz: summed over the 8 XCDs
    valu = tot["SQ_ACTIVE_INST_VALU"] * q / wave_steps * 2    # two waves per SIMD
    mfma = tot["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_steps
    coex = tot["SQ_VALU_MFMA_COEXEC_CYCLES"] / simd_steps
    lds = tot["SQ_LDS_IDX_ACTIVE"] / cu_steps
    bank = tot["SQ_LDS_BANK_CONFLICT"] / cu_steps
    lds_bytes = (tot["SQ_INSTS_LDS_LOAD_BANDWIDTH"] + tot["SQ_INSTS_LDS_STORE_BANDWIDTH"]) * 64 / cu_steps
    mops = tot["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / cu_steps
    pct = lambda x: f"{100 * x / step:.0f}%"
    lines = [
        "# Sequencer counters of `scan_mfma_kernel`, bidir307k", "",
        f"Workload: B={wl.B}, T={wl.T:,}, H={wl.H}, d={wl.d}, m={wl.m}, b={wl.b}; one `ttt_mlp_bidir` call: "
        f"{launches['n']} scan launches, {wg} workgroups of 8 waves each (one CU per head), "
        f"{2 * nblk:,} steps of 16 tokens per workgroup.", "",
        "Commands (repo root, MI355X), one run per counter set:", "",
    ]
    for i, p in enumerate(SQ_PASSES):
        lines.append(f"    rocprofv3 --pmc {p} --kernel-trace --output-format csv -d {dirs[i]} -o run -- "
                     "python3 -m test_rnn_layer_amd.profile_counters run")
    lines += [f"    python3 -m test_rnn_layer_amd.profile_counters summarize-sq " +
              " ".join(dirs[:len(SQ_PASSES)]), "",
              f"Kernel resources (kernel trace): scratch {row.get('Scratch_Size')} B per lane, LDS "
              f"{row.get('LDS_Block_Size')} B per workgroup (the build refuses any register spill).", "",
              f"A step takes {step:,.0f} cycles of a wave ({step / clock / 1e3:.2f} µs at the {clock:.2f} GHz that "
              f"GRBM_GUI_ACTIVE over the kernels' duration gives).", "",
              "| Per step | Value | Share of the step |", "|---|---|---|",
              f"| vector ALU busy, per SIMD (2 waves) | {valu:,.0f} cycles | {pct(valu)} |",
              f"| matrix core busy, per SIMD | {mfma:,.0f} cycles | {pct(mfma)} |",
              f"| of which beside a vector-ALU issue (co-execution) | {coex:,.0f} cycles | {pct(coex)} |",
              f"| LDS busy, per CU | {lds:,.0f} cycles | {pct(lds)} |",
              f"| of which bank-conflict stalls | {bank:,.0f} cycles | {pct(bank)} |",
              f"| LDS bytes moved, per CU | {lds_bytes / 1024:,.1f} KiB | — |",
              f"| wave waiting to issue (any / LDS), per wave | {tot['SQ_WAIT_INST_ANY'] * q / wave_steps:,.0f} / "
              f"{tot['SQ_WAIT_INST_LDS'] * q / wave_steps:,.0f} cycles | — |",
              f"| instructions per wave: vector ALU (incl. matrix) / matrix / LDS / scalar | "
              f"{tot['SQ_INSTS_VALU'] / wave_steps:.0f} / {tot['SQ_INSTS_MFMA'] / wave_steps:.0f} / "
              f"{tot['SQ_INSTS_LDS'] / wave_steps:.0f} / {tot['SQ_INSTS_SALU'] / wave_steps:.0f} | — |",
              f"| transcendental instructions per wave | {tot['SQ_INSTS_VALU_TRANS_F32'] / wave_steps:.1f} | — |",
              f"| bf16 matrix flops per CU (counter) | {mops / 1e6:.3f} M | — |", ""]
    out_md = out_md or os.path.join(ROOT, "profiles", "scan_mfma_bidir307k_sq_counters.md")
    open(out_md, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_stats(d: str, out_md: str | None = None):
    """Kernel-time table of a traced bench run (DIR/bench.json names the workload)."""
    from test_rnn_layer_amd import workloads as W
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(files[0])))
    bench = json.loads(open(os.path.join(d, "bench.json")).read().strip().splitlines()[-1])
    wname = bench["config"]["workload"]
    wl = W.WORKLOADS[wname]
    wl_arg = "" if wname == "bidir307k" else f" --workload {wname}"
    model = "TTT-Linear, d x d state" if wl.model == "linear" else "TTT-MLP"
    if wl.attn_seg > 0:
        model = f"segment attention (segments of {wl.attn_seg:,}, head width {wl.d}) + TTT-MLP"
    steps, warm = bench["steps"], bench["warmup"]
    calls = steps + warm
    tok = wl.B * wl.T
    lines = [
        f"# Kernel time, {wname} (one ttt_mlp_bidir call = both directions, each as chunked projection and scan "
        "launches)",
        "",
        f"Workload: {model}, B={wl.B}, T={wl.T:,}, H={wl.H}, d={wl.d}, m={wl.m}, b={wl.b}, bf16 X/θ/Y, fp32 state; "
        f"{steps} timed + {warm} warm-up calls under the trace.", "",
        "Commands (repo root, MI355X):", "",
        f"    mkdir -p {d} && rocprofv3 --kernel-trace --stats --output-format csv -d {d} -o run -- "
        f"python3 bench.py{wl_arg} --steps {steps} --warmup {warm} --no-cpu-baseline > {d}/bench.json",
        f"    python3 -m test_rnn_layer_amd.profile_counters summarize-stats {d}", "",
        "| Kernel | Launches | Average per launch | Per call | Share of kernel time |", "|---|---|---|---|---|",
    ]
    for r in rows:
        name = r["Name"].replace("ttt::(anonymous namespace)::", "")
        n = int(r["Calls"])
        lines.append(f"| `{name}` | {n} | {float(r['AverageNs']) / 1e6:.3f} ms | "
                     f"{float(r['TotalDurationNs']) / 1e6 / calls:.2f} ms | {float(r['Percentage']):.1f}% |")
    rf = bench["roofline"]
    if wl.attn_seg > 0:
        lines[0] = (f"# Kernel time, {wname} (one ttt_hybrid_block call: attention projections, segment attention "
                    "over segments of {:,} tokens, output projection, then the bidirectional TTT-MLP layer)"
                    .format(wl.attn_seg))
        what = (f"the attention's launches averaged {rf['avg_launch_ms']:.3f} ms from HIP events, "
                f"{rf['flops_per_launch'] / 1e12:.2f} TFLOP each, {rf['achieved']:.1f} TFLOP/s. The attention and "
                "its projections run before the TTT layer (it needs their output); inside the TTT layer the "
                "projection runs on a second stream beside the scan.")
        out_default = os.path.join(ROOT, "profiles", f"segment_attention_{wname}_stats.md")
    elif bench["config"]["scan_kernel"].endswith("mfma"):
        what = (f"the scan's launches averaged {rf['avg_launch_ms']:.3f} ms from HIP events on their stream, "
                f"{rf['flops_per_launch'] / 1e9:.1f} GFLOP each, {rf['achieved']:.1f} TFLOP/s. The projection runs "
                "on a second stream beside the scan; the call's time is that of the longer stream plus what cannot "
                "overlap (the first projection chunk of each direction, the last scan chunk).")
        out_default = os.path.join(ROOT, "profiles", f"{bench['config']['scan_kernel']}_proj_tiles_{wname}_stats.md")
    else:
        lines[0] = (f"# Kernel time, {wname} (one ttt_mlp_bidir call = both directions, each a projection of the "
                    "whole sequence, then one scan launch)")
        what = (f"the scan's launches averaged {rf['avg_launch_ms']:.3f} ms from HIP events on their stream, "
                f"{rf['flops_per_launch'] / 1e12:.2f} TFLOP each, {rf['achieved']:.2f} TFLOP/s. Each direction "
                "projects all its tokens, then scans them.")
        out_default = os.path.join(ROOT, "profiles", f"{bench['config']['scan_kernel']}_{wname}_stats.md")
    lines += ["", f"The bench line of the same run: {bench['ms_per_step']:.2f} ms per call "
              f"({bench['value'] / 1e6:.3f} M tokens/s, {100 * bench['layer_roofline']['frac']:.1f}% of the "
              f"roofline R = {bench['layer_roofline']['R_ms']:.2f} ms); " + what,
              f"Tokens per call: {tok:,} (both directions over every token)."]
    out_md = out_md or out_default
    open(out_md, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_backward(d: str, out_md: str | None = None):
    """Kernel-time table of a traced `bench.py --backward` run (DIR/bench.json)."""
    from test_rnn_layer_amd import workloads as W
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(files[0])))
    bench = json.loads(open(os.path.join(d, "bench.json")).read().strip().splitlines()[-1])
    wname = bench["config"]["workload"]
    wl = W.WORKLOADS[wname]
    steps, warm = bench["steps"], bench["warmup"]
    calls = steps + warm
    wl_arg = "" if wname == "bidir307k" else f" --workload {wname}"
    lines = [
        f"# Kernel time, backward of the bidirectional layer, {wname} (one ttt_mlp_bidir_backward call)", "",
        f"Workload: B={wl.B}, T={wl.T:,}, H={wl.H}, d={wl.d}, m={wl.m}, b={wl.b}, bf16 X/θ, fp32 arithmetic and "
        f"gradients; {steps} timed + {warm} warm-up calls under the trace.  One call: both forward passes again "
        "(projection, then the scan that keeps a checkpoint every 32 mini-batches: `scan_fwd_f32_kernel<false>`, "
        "fp32 matrix cores), then per direction windows of 16 checkpoint segments from the last: the first "
        "replayed on the call's stream (`scan_fwd_f32_kernel<true>`, one workgroup per head and segment), each "
        "later one on the library's second stream beside the walk of the window before, one segment per launch; "
        "each window walked by the backward scan (`scan_backward_split_kernel`, four workgroups per head, one "
        "cooperative launch per window; a clearing kernel zeroes dQ|dK|dV, the second dQ|dK buffer and the "
        "exchange entries per direction, a small kernel adds the second buffer in after the walk), the dalpha "
        "reduction, the exact three-part bf16 split of dQ|dK|dV and the two gradient GEMMs (dX, dθ; rocBLAS, "
        "bf16 operands, fp32 accumulation).", "",
        "Commands (repo root, MI355X):", "",
        f"    mkdir -p {d} && rocprofv3 --kernel-trace --stats --output-format csv -d {d} -o run -- "
        f"python3 bench.py --backward{wl_arg} --steps {steps} --warmup {warm} --no-cpu-baseline > {d}/bench.json",
        f"    python3 -m test_rnn_layer_amd.profile_counters summarize-backward {d}", "",
        "| Kernel | Launches | Average per launch | Per call | Share of kernel time |", "|---|---|---|---|---|",
    ]
    for r in rows:
        name = r["Name"].replace("ttt::(anonymous namespace)::", "")
        lines.append(f"| `{name}` | {int(r['Calls'])} | {float(r['AverageNs']) / 1e6:.3f} ms | "
                     f"{float(r['TotalDurationNs']) / 1e6 / calls:.1f} ms | {float(r['Percentage']):.1f}% |")
    rf = bench["roofline"]
    lines += ["", f"The bench line of the same run: {bench['ms_per_step']:.0f} ms per call "
              f"({bench['value']:,.0f} tokens/s); the backward scan's launches averaged {rf['avg_launch_ms']:.2f} ms "
              f"from HIP events, {rf['flops_per_launch'] / 1e9:.1f} GFLOP each (algorithmic, replay excluded), "
              f"{rf['achieved']:.2f} TFLOP/s = {100 * rf['frac']:.1f}% of the fp32 peak.  Kernel time per call "
              "(HIP events): " + ", ".join(f"{k.replace('_', ' ')} {v:.0f} ms"
                                            for k, v in bench.get("kernel_ms_per_step", {}).items()) + "."]
    out_md = out_md or os.path.join(ROOT, "profiles", f"scan_backward_{wname}_stats.md")
    open(out_md, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    sys.path.insert(0, ROOT)
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        run(*sys.argv[2:3])
    elif len(sys.argv) >= 4 and sys.argv[1] == "summarize":
        summarize(sys.argv[2], sys.argv[3])
    elif len(sys.argv) == 3 and sys.argv[1] == "summarize-stats":
        summarize_stats(sys.argv[2])
    elif len(sys.argv) == 3 and sys.argv[1] == "summarize-backward":
        summarize_backward(sys.argv[2])
    elif len(sys.argv) >= 3 and sys.argv[1] == "summarize-sq":
        summarize_sq(sys.argv[2:])
    else:
        print(__doc__)
        sys.exit(2)


