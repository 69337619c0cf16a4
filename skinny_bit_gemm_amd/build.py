"""Build libqlin.so and the measurement aid libqlin_probe.so (gfx950 only)
in-tree with hipcc.

Usage: python -m skinny_bit_gemm_amd.build   (or call build()).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqlin.so")
PROBE_LIB = os.path.join(HERE, "libqlin_probe.so")

ARCH = "gfx950"
# Packed fp32 VALU ops are disabled for all device code.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-munsafe-fp-atomics",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument"]
SOURCES = ["qlin_gemm_fp8.hip", "qlin_gemm_i8.hip", "qlin_gemm_block.hip", "qlin_kernels.hip",
           "qlin_api.cpp", "qlin_table.cpp"]
PROBE_SOURCES = ["qlin_probe.hip"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(hipcc, srcs, verbose):
    """Compile sources in parallel into OUT_DIR; returns the object paths."""
    objs, procs = [], []
    for src in srcs:
        obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        text = "\n".join(l for l in text.splitlines()
                         if "packed-fp32-ops" not in l and l.strip() != "1 warning generated.")
        if text.strip() and (verbose or p.returncode != 0):
            print(text, file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    return objs


def _link(hipcc, objs, lib, libs=()):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs, *libs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source and link libqlin.so (and the measurement aid
    libqlin_probe.so); returns the path of libqlin.so."""
    hipcc = _hipcc()
    os.makedirs(OUT_DIR, exist_ok=True)
    objs = _compile(hipcc, SOURCES + PROBE_SOURCES, verbose)
    _link(hipcc, objs[:len(SOURCES)], LIB, ["-ldl"])
    _link(hipcc, objs[len(SOURCES):], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
