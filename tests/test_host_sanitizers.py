"""Host C++ of the library under AddressSanitizer and UndefinedBehavior-
Sanitizer: tests/host/codebook_check.cpp linked with the codebook source,
built with g++ and run on the CPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_nf4_quantized_14_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_codebook_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "codebook_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host", "codebook_check.cpp"),
           os.path.join(CSRC, "codebook.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr
    # verify_asan_link_order=0: the sanitizer runtime need not be the first
    # library when the environment preloads another one
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120,
                         env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.strip() == "ok"
