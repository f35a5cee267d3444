"""Host-only code of the library under the address and undefined-behaviour
sanitizers, on the CPU: the descriptor checks of flashhead_prepare, the
cluster table's permutation check and inverse, and the INT4 centroid
quantizer (two_stage_retrieval_amd/csrc/fh_host.cpp, the same source the
library links).  tests/host/host_checks.cpp holds the checks."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _build(tmp_path, flags):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "host_checks")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *flags,
           "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "host", "host_checks.cpp"),
           os.path.join(ROOT, "two_stage_retrieval_amd", "csrc", "fh_host.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout
    return int(r.stdout.split()[1])


def test_host_code_under_asan_ubsan(tmp_path):
    exe = _build(tmp_path, ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"])
    assert _run(exe) > 1000


def test_host_code_plain_build(tmp_path):
    # the same checks without instrumentation, at the library's optimisation
    exe = _build(tmp_path, ["-O3", "-Wall", "-Werror"])
    assert _run(exe) > 1000
