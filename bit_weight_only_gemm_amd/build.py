"""Build the HIP library ``libw4a16.so`` in-tree for gfx950.

Every source is compiled with hipcc to an object under ``_build/`` (in
parallel), then linked into ``bit_weight_only_gemm_amd/libw4a16.so``.  Flags:
-O3, no fast-math and no flush-to-zero (fp16/bf16 subnormals must survive the
exact dequantization), no FP contraction (the dequant and epilogue round where
the definition says), and packed-fp32 instructions disabled.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libw4a16.so")
SOURCES = ["api.hip", "quant.hip", "gemm.hip", "gemm_b3.hip", "gemm_b8.hip", "prefill.hip",
           "prefill_b3.hip", "prefill_b8.hip", "measure.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


# Per-source flags.  The decode kernels keep their few accumulator tiles in
# ordinary VGPRs (MFMA with VGPR destination): with accumulation registers the
# compiler copies them back to VGPRs after every tile.  The prefill kernel's
# 256 accumulators need the accumulation registers and keeps the default.
_DECODE = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
EXTRA = {"gemm.hip": _DECODE, "gemm_b3.hip": _DECODE, "gemm_b8.hip": _DECODE}


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
