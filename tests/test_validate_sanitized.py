"""The library's host-side argument validation (csrc/validate.hpp), built with
g++ under AddressSanitizer and UndefinedBehaviorSanitizer and run over every
error path and a grid of extreme sizes (tests/validate_sanitized.cpp).  Any
sanitizer report aborts the driver (-fno-sanitize-recover), so a signed
overflow or out-of-bounds access in the validation arithmetic fails here.
No GPU is involved: validate.hpp is plain C++.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is not installed")
def test_validation_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "validate_sanitized"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-Wall", "-Werror",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "swiglu_mlp_fwd_amd", "csrc"),
           os.path.join(HERE, "validate_sanitized.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"build failed:\n{r.stderr}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, f"sanitized run failed:\n{r.stdout}\n{r.stderr}"
    assert "validate: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
