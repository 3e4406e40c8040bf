"""Host C++ of the library under AddressSanitizer and UndefinedBehavior-
Sanitizer, built with g++ and run on the CPU: tests/host/codebook_check.cpp
linked with the codebook source, and tests/host/plan_check.cpp linked with
the planning source (tile choice, the split of a ragged last wave, rank
stream and skinny plans, workspace layouts).  tests/host/quotient_check.cpp
checks, on its own, the block-scaled division that the 8-bit AdamW kernel
uses to encode its states (same E4M3 codes as IEEE division)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_nf4_quantized_14_amd", "csrc")


def _build_and_run(tmp_path, check_src, lib_src, sanitize=True):
    exe = tmp_path / os.path.splitext(os.path.basename(check_src))[0]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-ffp-contract=off"]
    if sanitize:
        cmd += ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    cmd += ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
            os.path.join(ROOT, "tests", "host", check_src)]
    if lib_src:
        cmd.append(os.path.join(CSRC, lib_src))
    cmd += ["-o", str(exe)]
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


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_codebook_under_asan_and_ubsan(tmp_path):
    _build_and_run(tmp_path, "codebook_check.cpp", "codebook.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_plans_and_layouts_under_asan_and_ubsan(tmp_path):
    _build_and_run(tmp_path, "plan_check.cpp", "plan.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_block_scaled_quotient_matches_ieee_codes(tmp_path):
    # plain build: 2.4e7 quotients, no sanitizer needed for the arithmetic
    _build_and_run(tmp_path, "quotient_check.cpp", None, sanitize=False)
