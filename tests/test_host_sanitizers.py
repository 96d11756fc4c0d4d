"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

A build of the same sources with the sanitizers on the host pass only (device code is compiled as
usual and never runs here) is loaded in a child process with the clang ASan runtime preloaded, and
the CPU tests that drive the host logic -- argument and shape checks of every entry point, stage
planning and its byte counts, the placement planner against exhaustive search -- run against it.
Any sanitizer report fails the test.  No GPU is needed.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

from pipeline_stage_decoder_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    rt = B.asan_runtime()
    if not rt:
        pytest.skip("the clang ASan runtime is not installed")
    lib = B.build_host_sanitized(str(tmp_path))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms, "host code is not instrumented"
    preload = rt + (":" + os.environ["LD_PRELOAD"] if os.environ.get("LD_PRELOAD") else "")
    env = dict(os.environ, LD_PRELOAD=preload, PSD_STAGE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi_host.py", "tests/test_placement.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
