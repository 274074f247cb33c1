"""Build libnvfp4.so (gfx950) in-tree with hipcc.

Usage: python -m bit_gemm_amd.build [--jobs N]

Every HIP source is compiled for gfx950 only, without FMA contraction (the
quantizer's fp32 steps are specified one rounding at a time) and without
packed-fp32 instructions; the objects are linked into
bit_gemm_amd/libnvfp4.so next to this file.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libnvfp4.so")
SOURCES = ["quantize.hip", "dequant.hip", "gemm_skinny.hip", "gemm_tiled.hip", "gptq.hip", "act_quant.hip", "gemm_dx.hip", "selftest.hip", "stream.hip", "noalloc.hip", "hessian.hip",
           "api.cpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


COMMON = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


# The GEMM sources once more with one tensor scale per group of stacked
# matrices (namespace nvfp4::grouped, for nvfp4_w4a16_gemm_grouped).
VARIANTS = [("gemm_skinny.hip", "gemm_skinny_grouped.o", ["-DNVFP4_GROUPED=1"]),
            ("gemm_tiled.hip", "gemm_tiled_grouped.o", ["-DNVFP4_GROUPED=1"])]


def _compile(job) -> str:
    src, obj_name, defs = job if isinstance(job, tuple) else (job, os.path.splitext(job)[0] + ".o", [])
    obj = os.path.join(BUILD, obj_name)
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *COMMON, *defs, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 6, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    # the two slowest compiles (and their grouped variants) first
    order = ["gemm_skinny.hip", VARIANTS[0], "gemm_tiled.hip", VARIANTS[1]] + \
        [s for s in SOURCES if s not in ("gemm_skinny.hip", "gemm_tiled.hip")]
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, order))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=min(6, os.cpu_count() or 1))
    args = ap.parse_args(argv)
    build(args.jobs, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
