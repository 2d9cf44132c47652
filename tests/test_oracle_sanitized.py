"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only): every function on small seeded shapes, with every array
allocated at exactly its documented size, plus refused bad ids.  A second
build plants a one-element-short output array and must be stopped by the
sanitizer, which shows that the check can fail."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "oracle_sanitize_check.c")
FLAGS = ["-std=c11", "-O1", "-g", "-ffp-contract=off", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _build(tmp_path, src, name):
    exe = str(tmp_path / name)
    r = subprocess.run(["gcc", *FLAGS, src, "-lm", "-o", exe], capture_output=True, text=True, timeout=120)
    if r.returncode != 0 and "sanitize" in r.stderr:
        pytest.skip("gcc has no sanitizer runtime here: " + r.stderr[-200:])
    assert r.returncode == 0, r.stderr
    return exe


def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    exe = _build(tmp_path, SRC, "oracle_san")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
    assert "runtime error" not in r.stderr


def test_sanitizer_stops_a_planted_overflow(tmp_path):
    text = open(SRC).read()
    short = "o.fan_src = alloc(Tk ? Tk - 1 : 0, sizeof(int32_t));"
    planted = text.replace("o.fan_src = alloc(Tk, sizeof(int32_t));", short)
    planted = planted.replace('#include "../../oracle/oracle.c"',
                              '#include "' + os.path.join(ROOT, "oracle", "oracle.c") + '"')
    assert short in planted
    src = tmp_path / "planted.c"
    src.write_text(planted)
    exe = _build(tmp_path, str(src), "planted")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=ENV)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
