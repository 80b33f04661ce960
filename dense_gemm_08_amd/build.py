"""Build step for libdense_gemm.so (hipcc, gfx950 only).

``python -m dense_gemm_08_amd.build`` compiles ``csrc/plan.cpp`` (host-side
argument checks and launch planning, plain C++), ``csrc/dense_gemm.hip`` (the
FP16/BF16 entry points, kernels in ``gemm_kernel.h``), ``csrc/ladder.hip``
(the optimisation-step kernels) and ``csrc/gemm_mx.hip`` (the FP8
block-scaled product, kernels in ``gemm_mx_kernel.h``) into
``dense_gemm_08_amd/libdense_gemm.so`` in place.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", n)
        for n in ("plan.cpp", "dense_gemm.hip", "ladder.hip", "gemm_mx.hip")]
OUT = os.path.join(HERE, "libdense_gemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from forming packed FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def build(extra=None, out=OUT, verbose=False) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + list(extra or []) + [
        "-I", os.path.join(ROOT, "include"),
        "-I", os.path.join(HERE, "csrc"),
    ] + SRCS + [
        "-o", tmp,
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(extra=sys.argv[1:], verbose=True))
