"""Workspace ownership bookkeeping on the host (tests/native/ledger_test.cpp over csrc/ledger.h).

A link call reads its plan's tables from the workspace and writes split partials and rotated
keys there, so pic_link_attend and pic_link_decode check that the workspace region still holds
their plan: an upload of another plan into any overlapping byte ends that claim. Built with g++
under the address and undefined-behaviour sanitizers."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "position_independent_kv_legolink_amd", "csrc")


def test_workspace_ledger(tmp_path):
    if not shutil.which("g++"):
        pytest.skip("g++ missing")
    exe = str(tmp_path / "ledger_test")
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-I", CSRC, os.path.join(ROOT, "tests", "native", "ledger_test.cpp"), "-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
