"""Build step: compiles the HIP library (gfx950) in-tree.

    python -m moe_expert_token_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_shuffle.so")
SOURCES = [os.path.join(CSRC, f) for f in ("abi.hip", "shuffle_kernels.hip")]
ARCH = os.environ.get("MOE_SHUFFLE_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(out: str = LIB, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp, *SOURCES]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(extra=sys.argv[1:]))
