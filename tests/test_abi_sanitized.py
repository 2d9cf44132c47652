"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
on the CPU: every source is rebuilt with the sanitizers on the host side
only (device code unchanged), and the C host check (argument validation,
workspace sizes, error strings, the reference copy's checks; no device
work) runs against it.  Any report fails the test."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CSRC = os.path.join(ROOT, "moe_expert_token_amd", "csrc")


def test_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("no ROCm toolchain")
    rt = subprocess.run([CLANG, "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("clang has no ASan runtime here")
    from moe_expert_token_amd import build
    objs, procs = [], []
    for src in build.SOURCES:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [HIPCC, f"--offload-arch={build.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
        objs.append(obj)
    for p in procs:
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, out.decode()[-2000:]
    lib = str(tmp_path / "libmoe_shuffle_asan.so")
    subprocess.run([HIPCC, f"--offload-arch={build.ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", lib, *objs],
                   check=True, capture_output=True, timeout=300)
    exe = str(tmp_path / "abi_host_check_asan")
    subprocess.run([CLANG, "-std=c99", "-g", "-fsanitize=address,undefined", "-shared-libsan",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_host_check.c"),
                    lib, "-Wl,-rpath," + str(tmp_path), "-o", exe], check=True, capture_output=True, timeout=300)
    env = dict(os.environ, LD_LIBRARY_PATH=os.path.dirname(rt), ASAN_OPTIONS="detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
