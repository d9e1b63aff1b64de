"""HBM traffic of the scan kernel from rocprofv3 counters.

    # one counter per run (each run: a known-size copy, then one layer call)
    rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d DIR_F -o run -- \
        python3 -m test_rnn_layer_amd.profile_counters run
    rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d DIR_W -o run -- \
        python3 -m test_rnn_layer_amd.profile_counters run
    python3 -m test_rnn_layer_amd.profile_counters summarize DIR_F DIR_W

`run` makes one device-to-device copy of COPY_BYTES (the runtime's copy
kernel reads and writes exactly that many bytes), then one ttt_mlp_bidir
call of the workload.  `summarize` scales each counter by what it read for
the copy, and writes the scan kernel's bytes per launch into
profiles/scan_traffic.json, keyed by kernel, with a digest of the scan
sources so that a later kernel change invalidates it.
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
KERNELS = {"scan_mfma": "scan_mfma_kernel", "scan_generic": "scan_generic_kernel", "scan_coop": "scan_coop_kernel",
           "projection": "proj_tiles_kernel"}
# the sources each kernel is built from: its counters are stale once any of them changes
KERNEL_SOURCES = {"scan_mfma": ["scan_mfma.hip", "mfma_common.h", "internal.h"],
                  "scan_generic": ["generic.hip", "internal.h"],
                  "scan_coop": ["scan_coop.hip", "internal.h"],
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
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    sys.path.insert(0, ROOT)
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        run(*sys.argv[2:3])
    elif len(sys.argv) >= 4 and sys.argv[1] == "summarize":
        summarize(sys.argv[2], sys.argv[3])
    else:
        print(__doc__)
        sys.exit(2)
