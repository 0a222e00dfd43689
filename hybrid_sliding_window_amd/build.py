"""Build libhsw.so (the C-ABI library of hand-written gfx950 HIP kernels) in
place, next to this file, and libhsw_checked.so, the same sources built with
HSW_CHECK_DEVICE=1 (device-resident arguments checked on the device before
each call's kernels run).  libhsw_measure.so holds measurement-only kernels
(measure/*.hip) that bench.py times beside the path's own; nothing of the
path uses it.

    python -m hybrid_sliding_window_amd.build

Each .hip source is compiled separately (in parallel) for --offload-arch=gfx950
and linked into one shared library per build.  Packed-fp32 instruction
selection is disabled for the device code (some of those forms are not
trusted here).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libhsw.so")
CHECKED_LIB = os.path.join(HERE, "libhsw_checked.so")
MEASURE_LIB = os.path.join(HERE, "libhsw_measure.so")
MEASURE_SRC = os.path.join(HERE, "measure")
BUILD_DIR = os.path.join(HERE, "_build")
CHECKED_BUILD_DIR = os.path.join(HERE, "_build_checked")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# The MFMA prefill kernels take no NaN inputs on their hot path (masked logits
# are -inf, never NaN), so fmax needs no quieting of its operands: without
# this, every max over logits costs an extra canonicalising instruction.
RELAXED_NAN = {"swa_prefill.hip", "full_prefill.hip"}
RELAXED_NAN_FLAGS = ["-fno-honor-nans", "-mno-amdgpu-ieee"]


def _compile(src: str, build_dir: str, checked: bool) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    extra = RELAXED_NAN_FLAGS if os.path.basename(src) in RELAXED_NAN else []
    if checked:
        extra = extra + ["-DHSW_CHECK_DEVICE=1"]
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, checked: bool = True) -> str:
    """Compile and link libhsw.so, (checked=True) libhsw_checked.so, and
    libhsw_measure.so."""
    builds = [(BUILD_DIR, LIB, False)] + ([(CHECKED_BUILD_DIR, CHECKED_LIB, True)] if checked else [])
    srcs = sources()
    msrcs = sorted(glob.glob(os.path.join(MEASURE_SRC, "*.hip")))
    jobs = []
    for d, _, chk in builds:
        os.makedirs(d, exist_ok=True)
        jobs += [(src, d, chk) for src in srcs]
    jobs += [(src, BUILD_DIR, False) for src in msrcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    n = len(srcs)
    for i, (_, lib, _) in enumerate(builds):
        _link(objs[i * n:(i + 1) * n], lib)
        if verbose:
            print("built", lib)
    if msrcs:
        _link(objs[len(builds) * n:], MEASURE_LIB)
        if verbose:
            print("built", MEASURE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
