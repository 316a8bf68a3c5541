"""Sanitizer builds on the CPU: the C oracle under AddressSanitizer +
UndefinedBehaviorSanitizer and under ThreadSanitizer (its thread pool), and
the library's host-side argument layer under AddressSanitizer +
UndefinedBehaviorSanitizer with stub launchers (no GPU).  The drivers are in
tests/sanitize/; a memory error, undefined behaviour or data race aborts the
driver, and a wrong result makes it exit non-zero."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIP_INCLUDE = "/opt/rocm/include"


def _build_and_run(cmd, exe):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
    for word in ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer"):
        assert word not in r.stderr, r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
@pytest.mark.parametrize("san", ["address,undefined", "thread"])
def test_oracle_under_sanitizers(tmp_path, san):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-Wall", "-ffp-contract=off", f"-fsanitize={san}",
           "-fno-sanitize-recover=all", "-o", exe, os.path.join(ROOT, "oracle", "bole_oracle.c"),
           os.path.join(SAN, "oracle_driver.c"), "-lpthread", "-lm"]
    _build_and_run(cmd, exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(HIP_INCLUDE),
                    reason="g++ or the HIP headers not found")
def test_abi_argument_layer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-Wall", "-x", "c++", "-D__HIP_PLATFORM_AMD__",
           "-I", HIP_INCLUDE, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "linear_attention_tree_amd", "csrc"),
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", exe,
           os.path.join(SAN, "abi_driver.cpp")]
    _build_and_run(cmd, exe)
