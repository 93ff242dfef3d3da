"""Build libcanon.so (HIP for gfx950) in-tree with hipcc, and the test
library of a caller-defined operator (tests/user_op).

Usage: python -m scan_canonical_reduce_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libcanon.so")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build", "libcanon")

SOURCES = [
    "api.cpp", "reduce.hip", "scan.hip", "scan_with_init.hip", "scan_wide.hip",
    "scan_wide_init.hip", "scan_lane.hip", "scan_lane_init.hip", "scan_rows.hip", "scan_ip.hip",
    "scan_ip1.hip", "scan_ip1_narrow_f64.hip", "scan_ip1_narrow_f32.hip",
    "ops_mul_f64.hip", "ops_mul_f32.hip", "ops_min_f64.hip", "ops_min_f32.hip",
    "ops_max_f64.hip", "ops_max_f32.hip", "scan_noalloc.cpp",
]

# -ffp-contract=off: no FMA contraction; no fast-math; subnormals kept (no
# flush to zero in device code, float included); packed FP32 disabled.
HIPFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero", "-Xclang", "-target-feature",
    "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [_hipcc(), *HIPFLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


# Libraries built from canon_user_op.hpp with a caller-defined operator:
# (source, output), relative to the repository root.  The skew operator is
# the one the GPU tests of caller-defined operators load.
ROOT = os.path.dirname(HERE)
USER_OP_LIBS = [("tests/user_op/skew_op.hip", "tests/user_op/libcanon_skew.so")]

# The benchmark's bandwidth probes (their own library, not libcanon's ABI).
PROBE_LIB = ("scan_canonical_reduce_amd/csrc/bw_probe.hip",
             "scan_canonical_reduce_amd/libcanon_bwprobe.so")


def _build_user_op(pair) -> str:
    src, out = (os.path.join(ROOT, p) for p in pair)
    tmp = out + ".tmp"
    cmd = [_hipcc(), *HIPFLAGS, "-shared", "-I", os.path.join(ROOT, "include"), "-I", CSRC, src,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        user = [ex.submit(_build_user_op, p) for p in USER_OP_LIBS]  # longest first
        user.append(ex.submit(_build_user_op, PROBE_LIB))
        objs = list(ex.map(_compile, srcs))
        for f in user:
            f.result()
    tmp = OUT + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
