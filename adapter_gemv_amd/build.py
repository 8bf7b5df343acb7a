"""Build libsgmv.so in-tree with hipcc for gfx950.

    python -m adapter_gemv_amd.build          # compile and link
    python -m adapter_gemv_amd.build --asm    # also write the gfx950 assembly
    python -m adapter_gemv_amd.build --phases # profiling variant with phase timestamps

Every HIP source is compiled with packed FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libsgmv.so")
PHASES_LIB_PATH = os.path.join(PKG, "libsgmv_phases.so")
ARCH = "gfx950"

SOURCES = ["sgmv_segments.cpp", "sgmv_cache.cpp", "sgmv_kernels.hip", "sgmv_decode.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}",
          "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsgmv)")


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    lines = [ln for ln in res.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def build(asm: bool = False, verbose: bool = False, phases: bool = False) -> str:
    """Compile every source and link libsgmv.so; returns the library path.  phases=True
    builds the profiling variant libsgmv_phases.so instead, whose one-launch kernels write
    per-phase timestamps (-DSGMV_PHASE_STAMPS; bench.py --phases reads them)."""
    hipcc = _hipcc()
    bdir = os.path.join(BUILD_DIR, "phases") if phases else BUILD_DIR
    out = PHASES_LIB_PATH if phases else LIB_PATH
    flags = COMMON + (["-DSGMV_PHASE_STAMPS"] if phases else [])
    os.makedirs(bdir, exist_ok=True)
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        jobs.append([hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    if asm:
        for src in SOURCES:
            if src.endswith(".hip"):
                jobs.append([hipcc, *COMMON, "--cuda-device-only", "-S", os.path.join(CSRC, src),
                             "-o", os.path.join(BUILD_DIR, src.replace(".hip", ".gfx950.s"))])
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o:
                print(o)
    tmp = out + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, out)
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--asm", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--phases", action="store_true",
                    help="build the phase-timestamp profiling variant libsgmv_phases.so")
    args = ap.parse_args(argv)
    print(build(asm=args.asm, verbose=args.verbose, phases=args.phases))
    return 0


if __name__ == "__main__":
    sys.exit(main())
