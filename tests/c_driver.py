"""Builds and runs tests/c/abi_gpu_drive.c, a plain C program that drives
the library on the GPU with HIP allocations of its own (no Python in the
data path, no PyTorch).  Test infrastructure: compiled by
__graft_entry__.build() next to its source, linked to the in-tree library."""

import os
import subprocess

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "abi_gpu_drive.c")
EXE = os.path.join(ROOT, "tests", "c", "abi_gpu_drive")


def compile_cmd(exe: str = EXE, extra=()) -> list:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return ["gcc", "-std=gnu11", "-O2", *extra, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
            "-I", os.path.join(rocm, "include"), SRC, "-o", exe,
            "-L", os.path.join(ROOT, "moe_expert_token_amd"), "-lmoe_shuffle",
            "-L", os.path.join(rocm, "lib"), "-lamdhip64",
            "-Wl,-rpath,$ORIGIN/../../moe_expert_token_amd", "-Wl,-rpath," + os.path.join(rocm, "lib")]


def build(exe: str = EXE) -> str:
    subprocess.run(compile_cmd(exe), check=True)
    return exe


def run(T, H, E, k, R, idx, x, w, ye=None, timeout=120):
    """Runs the driver on one batch (x, w, ye as float arrays whose values
    are exact in bf16); returns {name: array} of everything it printed."""
    if not os.path.exists(EXE):
        build()
    vals = [f"{T} {H} {E} {k} {R}", " ".join(str(int(v)) for v in np.asarray(idx).ravel()),
            " ".join(repr(float(v)) for v in np.asarray(x, np.float32).ravel()),
            " ".join(repr(float(v)) for v in np.asarray(w, np.float32).ravel())]
    if ye is None:
        vals.append("0")
    else:
        vals += ["1", " ".join(repr(float(v)) for v in np.asarray(ye, np.float32).ravel())]
    r = subprocess.run([EXE], input="\n".join(vals) + "\n", capture_output=True, text=True, timeout=timeout)
    out = {}
    for line in r.stdout.splitlines():
        name, *rest = line.split()
        if name in ("xr", "xe", "out"):
            out[name] = np.array([float(v) for v in rest], dtype=np.float32)
        elif name == "ERROR":
            out[name] = rest
        else:
            out[name] = np.array([int(v) for v in rest], dtype=np.int64)
    out["returncode"] = r.returncode
    out["stderr"] = r.stderr
    return out
