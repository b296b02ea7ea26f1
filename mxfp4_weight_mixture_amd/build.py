"""Builds libmxmoe.so in-tree with hipcc for gfx950.

    python -m mxfp4_weight_mixture_amd.build        (or build() from Python)

Every .hip file under csrc/ is compiled for gfx950 only, in parallel, then
linked into mxfp4_weight_mixture_amd/libmxmoe.so.  Packed-FP32 VALU ops are
disabled for the device code (-packed-fp32-ops): the compiler would otherwise
form v_pk_* fp32 instructions from ordinary float code.

Two measurement libraries are built beside it: libmxmoe_probe.so (probe/:
matrix-instruction issue rates, HBM stream read, 16 KB chunk streams) and
libmxmoe_phases.so, the same sources with the grouped GEMM's phase timers
compiled in (MXMOE_PHASE_TIMERS=1), which `bench.py --phases` loads.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmxmoe.so")
# measurement tooling (matrix-instruction issue rates, HBM stream read), a library of its own
# outside libmxmoe's ABI
PROBE_DIR = os.path.join(PKG, "probe")
PROBE_LIB = os.path.join(PKG, "libmxmoe_probe.so")
PHASES_LIB = os.path.join(PKG, "libmxmoe_phases.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
CXXFLAGS = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    "-I" + os.path.join(ROOT, "include"),
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmxmoe.so)")


def _compile(src: str, phases: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + (".phases.o" if phases else ".o"))
    cmd = [hipcc(), *CXXFLAGS, *(["-DMXMOE_PHASE_TIMERS=1"] if phases else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    gemm = os.path.join(CSRC, "gemm.hip")
    with cf.ThreadPoolExecutor(jobs + 1) as ex:
        phases_obj = ex.submit(_compile, gemm, True)
        objs = list(ex.map(_compile, srcs))
        phases_obj = phases_obj.result()

    def link(lib, lib_objs):
        tmp = lib + ".tmp"
        cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *lib_objs, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, lib)

    link(LIB, objs)
    gemm_obj = os.path.join(BUILD_DIR, "gemm.hip.o")
    link(PHASES_LIB, [o for o in objs if o != gemm_obj] + [phases_obj])
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc(), *CXXFLAGS, "-shared", *sorted(glob.glob(os.path.join(PROBE_DIR, "*.hip"))), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the probe failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print("built", LIB, "and the measurement libraries", PROBE_LIB, PHASES_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
