"""Ahead-of-time build of the HIP library ``libtg.so`` for gfx950.

Every source under ``csrc/`` is compiled with hipcc into ``_build/`` and
linked into ``tiled_dense_gemm_05_amd/libtg.so`` next to this file.  Run
``python tiled_dense_gemm_05_amd/build.py`` (the repository root's entry module calls it too);
it is a plain script so that it never imports the package it builds.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtg.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]

# Per-source flags.  The attention kernel's scores never hold NaN (masked keys
# are -inf): telling the compiler so lets fmaxf map to v_max3_f32 without
# first quieting each matrix-core result.
PER_FILE = {
    "attention.hip": ["-fno-honor-nans"],
}


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *PER_FILE.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        # the host pass does not know the packed-fp32 feature; keep other warnings
        lines = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln
                 and "not a recognized feature" not in ln]
        if any(ln.strip() for ln in lines):
            sys.stderr.write("\n".join(lines) + "\n")
    return obj


def build_library(extra: list[str] | None = None) -> str:
    """Compile every source and link libtg.so; returns its path."""
    extra = list(extra or [])
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_capi_bench()
    build_ceilings()
    return LIB


BENCH_SRC = os.path.join(HERE, "capi_bench.cpp")
BENCH_BIN = os.path.join(HERE, "tg_capi_bench")


def build_capi_bench() -> str:
    """The C++ timing program that calls the library through its C ABI only."""
    tmp = BENCH_BIN + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), BENCH_SRC,
           "-o", tmp, "-L", HERE, "-ltg", "-Wl,-rpath,$ORIGIN"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the C ABI benchmark failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, BENCH_BIN)
    return BENCH_BIN


CEIL_SRC = os.path.join(HERE, "ceilings.hip")
CEIL_BIN = os.path.join(HERE, "tg_ceilings")


def build_ceilings() -> str:
    """The program that measures the part's practical ceilings (matrix-core
    rate and clock on the workload's data, LDS read rates)."""
    tmp = CEIL_BIN + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", CEIL_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the ceilings program failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, CEIL_BIN)
    return CEIL_BIN


if __name__ == "__main__":
    print(build_library(sys.argv[1:]))
