"""Build libqproj.so (every HIP source under csrc/) for gfx950 with hipcc.

The library is built in-tree, next to this file, so that it travels with
the source tree.  Flags:
  --offload-arch=gfx950                  CDNA4 only
  -ffp-contract=off                      no silent FMA contraction (the
                                         quantizers round every step; the
                                         GEMMs ask for FMA explicitly)
  -fhip-fp32-correctly-rounded-divide-sqrt  IEEE binary32 division, which the
                                         code rounding relies on
  -target-feature -packed-fp32-ops       no packed-FP32 VALU instructions
Per file (FILE_FLAGS):
  gemv_w4a16.hip, gemm_int8.hip: -mllvm -amdgpu-mfma-vgpr-form
                                         MFMA results in ordinary VGPRs:
                                         these kernels fold every MFMA result
                                         with VALU FMAs, and the
                                         accumulator-register form costs a
                                         copy per value read
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libqproj.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

DEVICE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
]


FILE_FLAGS = {
    "gemv_w4a16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "gemm_int8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *DEVICE_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link libqproj.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
