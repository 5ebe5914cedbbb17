"""Build libgla.so (the HIP/gfx950 GLA library) in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only, in parallel, into
``_build/`` and linked into ``chunkwise_linear_rnn_gla_amd/libgla.so``.
Packed fp32 vector instructions are disabled for the device code
(``-packed-fp32-ops``); hipcc's host pass warns that it does not know that
feature, which is expected.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgla.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
]
# Per-source extras.  Most kernels keep their MFMA accumulators in ordinary
# VGPRs (no accumulator-register moves around every use of an accumulator).
EXTRA_FLAGS = {
    "gla_prep.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    # the recurrence's chunk body is one long block of LDS reads and MFMAs;
    # the ILP-oriented scheduler interleaves them far better than the default
    # occupancy-oriented one (one wave per SIMD runs there anyway)
    "gla_recur.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
    # the general gate's recurrence rescales and converts its state every
    # chunk: in accumulator registers each such access costs a move
    "gla_ggate.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    # the backward's state recurrences: accumulators read as operands every
    # chunk; the ILP scheduler helps its one wave per SIMD as it does the
    # forward's recurrence
    "gla_bwd_recur.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
    # dq and dk: the intra-chunk products' accumulators are scaled and summed
    # on the vector ALU right after the MFMAs
    "gla_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    extra = EXTRA_FLAGS.get(os.path.basename(src), [])
    cmd = [HIPCC, *CFLAGS, *extra, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-8000:]}")
    _check_no_scratch(src, r.stderr)
    return obj


def _check_no_scratch(src: str, remarks: str) -> None:
    """Every kernel must keep its working set in registers and LDS: a kernel
    that spills to scratch is rejected at build time."""
    name = None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            raise RuntimeError(f"{os.path.basename(src)}: kernel {name} uses "
                               f"{m.group(1)} bytes/lane of scratch (register spill)")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-8000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
