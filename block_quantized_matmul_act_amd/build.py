"""Build libkq.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["kq_api.cpp", "kq_quant.hip", "kq_gemm.hip", "kq_gemm_q4k.hip", "kq_gemm_ring.hip", "kq_gemm_tq.hip", "kq_gemv.hip", "kq_calib.hip"]
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no fast-math; no fp contraction outside explicit fmaf() calls, so the
    # activation quantizer's x*s is a single rounded multiply
    "-ffp-contract=off",
    # keep the compiler from emitting packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    # MFMA accumulators in ordinary VGPRs: the fold reads and writes them with
    # VALU instructions, and AGPR placement would add a copy per element
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source into libkq.so (always recompiles)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *(extra or []), "-x", "hip", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd, cwd=CSRC)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
