"""Builds the HIP library libttt_mlp.so for gfx950, in-tree.

    python -m test_rnn_layer_amd.build [-v] [--phase-marks]

hipcc cross-compiles without a GPU.  Every source is compiled on each call.
--phase-marks builds the measurement variant libttt_mlp_marks.so instead: the
same sources with TTT_PHASE_MARKS defined, whose scan kernels record the shader
clock at the phase boundaries of their steps (see csrc/phase_marks.h and
phase_profile.py).
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libttt_mlp.so")
MARKS_BUILD_DIR = os.path.join(PKG, "_build_marks")
MARKS_LIB_PATH = os.path.join(PKG, "libttt_mlp_marks.so")
SOURCES = ["api.hip", "generic.hip", "proj_mfma.hip", "scan_mfma.hip", "scan_linear.hip", "scan_coop.hip",
           "backward.hip", "backward_split.hip", "scan_fwd_f32.hip", "grad_gemm.hip", "attention.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from emitting packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"),
]


# kernels that must keep their whole working set in registers: the MFMA and
# cooperative scans and the backward's fp32 matrix-core forward pass hold the
# inner-model state in VGPRs for the whole sequence (and the linear scan counts
# its vector-memory instructions per
# step), the projection GEMM's accumulators and operands fill the register
# file (a spill there cost a fifth of its speed), and the split backward walk
# saved and reloaded its spilled registers through scratch memory around every
# product call (35.7 against 27.1 us a mini-batch), so a spilling build of any
# of them is refused.
NO_SPILL_SOURCES = {"scan_mfma.hip", "scan_linear.hip", "scan_coop.hip", "proj_mfma.hip", "scan_fwd_f32.hip",
                    "backward_split.hip"}


def _check_no_spill(src, remarks):
    spills = re.findall(r"VGPRs Spill: (\d+)", remarks) + re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", remarks)
    if not spills:
        raise RuntimeError(f"{src}: no resource-usage report from the compiler")
    if any(int(x) for x in spills):
        raise RuntimeError(f"{src}: the kernel spills registers to scratch:\n{remarks}")


# kernels whose matrix-core accumulation chains must stay on one instruction: a
# 16x16x32 result read as the accumulator of a 16x16x16 product a few
# instructions later gave wrong values on gfx950 (the compiler inserts no wait
# for it).  The build compiles these sources to assembly as well and refuses any
# product whose accumulator comes from a product of another instruction.
MFMA_CHAIN_SOURCES = {"scan_mfma.hip", "scan_linear.hip", "proj_mfma.hip", "attention.hip", "scan_fwd_f32.hip"}
_MFMA = re.compile(r"\s*(v_mfma\w*)\s+v\[(\d+):(\d+)\],\s*[^,]+,\s*[^,]+,\s*(?:v\[(\d+):(\d+)\]|\S+)")
_VDST = re.compile(r"\s*(?:v_|ds_read|global_load|buffer_load|scratch_load|flat_load)\S*\s+(?:v(\d+)|v\[(\d+):(\d+)\])")


def _vdst(line):
    m = _VDST.match(line)
    if not m or line.lstrip().startswith(("v_cmp", "v_readlane", "v_readfirstlane")):
        return None
    return (int(m.group(1)), int(m.group(1))) if m.group(1) else (int(m.group(2)), int(m.group(3)))


def _check_mfma_chains(src, asm_path, window=48):
    """Follows each matrix-core result until its registers are overwritten; a
    product of another instruction that takes it as accumulator is refused."""
    lines = [l.strip() for l in open(asm_path) if l.strip() and not l.strip().startswith((";", "."))]
    bad = []
    for i, line in enumerate(lines):
        m = _MFMA.match(line)
        if not m:
            continue
        d0, d1 = int(m.group(2)), int(m.group(3))
        for k in range(i + 1, min(i + 1 + window, len(lines))):
            if lines[k].endswith(":"):  # a label: the straight-line region ends
                break
            m2 = _MFMA.match(lines[k])
            if m2 and m2.group(4) is not None and int(m2.group(4)) <= d1 and int(m2.group(5)) >= d0:
                if m2.group(1) != m.group(1):
                    bad.append(f"{line}  ->  {lines[k]}")
                break
            dst = _vdst(lines[k])
            if dst is not None and dst[0] <= d1 and dst[1] >= d0:
                break
    if bad:
        raise RuntimeError(f"{src}: accumulator taken from a product of another matrix-core instruction:\n" +
                           "\n".join(bad))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = r.stdout
    src = os.path.basename(cmd[cmd.index("-c") + 1]) if "-c" in cmd else ""
    if r.returncode == 0 and "-S" in cmd:
        _check_mfma_chains(src, cmd[cmd.index("-o") + 1])
        src = ""
    if r.returncode == 0 and src in NO_SPILL_SOURCES and "-Rpass-analysis=kernel-resource-usage" in cmd:
        _check_no_spill(src, "\n".join(l for l in out.splitlines() if "remark" in l))
        out = "\n".join(l for l in out.splitlines() if "remark" not in l)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out:
        print(out)


def build(verbose: bool = False, phase_marks: bool = False) -> str:
    build_dir, lib_path = (MARKS_BUILD_DIR, MARKS_LIB_PATH) if phase_marks else (BUILD_DIR, LIB_PATH)
    flags = FLAGS + (["-DTTT_PHASE_MARKS=1"] if phase_marks else [])
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        # the measurement build keeps the library's checks off: its marks add a few live registers
        checked = src in NO_SPILL_SOURCES and not phase_marks
        extra = ["-Rpass-analysis=kernel-resource-usage"] if checked else []
        cmds.append([HIPCC, *flags, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
        if src in MFMA_CHAIN_SOURCES and not phase_marks:
            asm = os.path.join(build_dir, os.path.splitext(src)[0] + ".s")
            cmds.append([HIPCC, *flags, "--cuda-device-only", "-S", "-c", os.path.join(CSRC, src), "-o", asm])
    with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = lib_path + ".tmp"
    # rocBLAS runs the backward's two plain fp32 gradient GEMMs (grad_gemm.hip)
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-L/opt/rocm/lib", "-lrocblas",
          "-Wl,-rpath,/opt/rocm/lib"], verbose)
    shutil.move(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, phase_marks="--phase-marks" in sys.argv))
