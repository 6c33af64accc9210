"""The store, planner and C ABI built with the address and undefined-behaviour sanitizers.

tests/native/abi_fuzz.cpp drives the C ABI on metadata-only stores (no device) with seeded
random stores, chunks, requests and options, valid and invalid, and checks the exported plans'
invariants and the page accounting. The host sources are built with g++ (no device code; the
kernel launchers are test-only stubs that are never reached), so AddressSanitizer, its leak
checker and UBSan see every host allocation and access of the library.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "position_independent_kv_legolink_amd", "csrc")
ROCM = "/opt/rocm"


@pytest.fixture(scope="module")
def fuzzer(tmp_path_factory):
    if not shutil.which("g++") or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers are missing")
    exe = str(tmp_path_factory.mktemp("asan") / "abi_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "planner.cpp"), os.path.join(CSRC, "abi.cpp"),
           os.path.join(ROOT, "tests", "native", "launch_stubs.cpp"),
           os.path.join(ROOT, "tests", "native", "abi_fuzz.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_abi_fuzz_under_sanitizers(fuzzer, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([fuzzer, str(seed), "250"], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert r.stdout.startswith("ok:"), r.stdout
    plans = int(r.stdout.split(",")[1].split()[0])
    assert plans > 50, r.stdout
