"""Build step: compiles the HIP library (gfx950) in-tree.

    python -m moe_expert_token_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_shuffle.so")
SOURCES = [os.path.join(CSRC, f) for f in ("abi.hip", "plan.hip", "rows.hip", "reduce.hip", "combine_bwd.hip", "copy_ref.hip")]
ARCH = os.environ.get("MOE_SHUFFLE_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(out: str = LIB, extra=()) -> str:
    """Compiles every source to an object (in parallel), then links the
    shared library; `extra` flags go to every compile."""
    with tempfile.TemporaryDirectory() as tmpdir:
        procs, objs = [], []
        for src in SOURCES:
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src,
                   "-o", obj]
            procs.append((subprocess.Popen(cmd), cmd))
            objs.append(obj)
        failed = [cmd for p, cmd in procs if p.wait() != 0]
        if failed:
            raise subprocess.CalledProcessError(1, failed[0])
        tmp = out + ".tmp"
        subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(extra=sys.argv[1:]))
