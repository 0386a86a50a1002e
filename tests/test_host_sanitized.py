"""The library's host code (planner, validation, sizes, argument checks of the
compute calls) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer and driven by ``tests/host/host_fuzz.cpp`` over
seeded random arguments. Host code only: the kernel launchers are stubs, no
GPU is involved."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_code_under_sanitizers(tmp_path):
    exe = tmp_path / "host_fuzz"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "split_kv_flash_decode_amd", "csrc"),
           os.path.join(ROOT, "split_kv_flash_decode_amd", "csrc", "skv_host.cpp"),
           os.path.join(ROOT, "tests", "host", "host_fuzz.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    # (verify_asan_link_order=0: an environment may preload other libraries)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host fuzz ok" in r.stdout
