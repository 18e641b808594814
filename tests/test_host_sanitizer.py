"""The host planner (csrc/plan.cpp: layout validation, tile classification,
work lists, the backward's key lists) built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven by a seeded fuzz of layouts
(tests/c/plan_fuzz.cpp): packed videos, KV caches, KV ranges, last global
blocks, chunk-wise text prompts, broken layouts that must be refused, and
offsets at the 2 GiB tensor limits and next to INT32_MAX. Any out-of-bounds
access, use after free, leak, signed overflow or failed list check fails the
test. CPU only: g++, no HIP code is compiled or run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_causal_attention_flash_amd", "csrc")


@pytest.fixture(scope="module")
def fuzz_bin(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ and the ROCm headers are needed")
    out = str(tmp_path_factory.mktemp("asan") / "plan_fuzz")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + CSRC, os.path.join(CSRC, "plan.cpp"), os.path.join(ROOT, "tests", "c", "plan_fuzz.cpp"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return out


def test_planner_fuzz_under_asan_and_ubsan(fuzz_bin):
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([fuzz_bin, "400", "1000"], capture_output=True, text=True, env=env, timeout=600)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr
    assert " 0 failed checks" in res.stdout
