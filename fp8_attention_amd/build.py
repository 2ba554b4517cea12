"""Build libdm.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

Also builds the test-only probe of the FP8 matrix instructions
(tests/hip/libmfma_acc.so), which the GPU tests use to measure how the
instructions the kernels rely on accumulate; it is not part of libdm.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdm.so")
SOURCES = ["api.hip", "quantize.hip", "attn_fwd.hip", "attn_delta.hip", "attn_bwd.hip", "attn_dkdv_wide.hip",
           "attn_dq.hip", "attn_dq_wide.hip", "attn_dkdv128.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         # keep the compiler away from packed FP32 instructions on this target
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# Attention kernels: scores are finite or -inf by construction, so max
# reductions need no NaN canonicalisation (this lets them map onto v_max3_f32).
EXTRA = {src: ["-fno-honor-nans"]
         for src in ("attn_fwd.hip", "attn_delta.hip", "attn_bwd.hip", "attn_dkdv_wide.hip", "attn_dq.hip",
                     "attn_dq_wide.hip", "attn_dkdv128.hip")}
# The generic dK/dV kernel and the dQ kernels: keep MFMA results in VGPRs so the FP32
# softmax work on the score tiles does not shuttle them through AGPRs.  (The
# d_qk=192/d_v=128 dQ instance is built without it: the compiler fails on it; the
# d = 256 instances, one wave per SIMD, need the AGPRs for their accumulators.)
EXTRA["attn_bwd.hip"] += ["-mllvm", "--amdgpu-mfma-vgpr-form"]
EXTRA["attn_dq.hip"] += ["-mllvm", "--amdgpu-mfma-vgpr-form"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


PROBE_SRC = os.path.join(ROOT, "tests", "hip", "mfma_acc.hip")
PROBE_LIB = os.path.join(ROOT, "tests", "hip", "libmfma_acc.so")


def build_probe() -> str:
    """The test-only instruction probe (tests/hip/mfma_acc.hip -> tests/hip/libmfma_acc.so)."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PROBE_SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_probe()
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
