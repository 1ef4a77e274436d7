"""The walk lengths and key-split run counts shared by the host and the
kernels (csrc/ra_walk.h), checked on the CPU: walk_check.cpp compares them
with brute force from the visibility definition over a sweep of shapes,
masks and placements, and checks that the kernels' workgroup mapping covers
every run exactly once.  Built with g++ under AddressSanitizer and UBSan."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_walk_lengths_and_run_counts(tmp_path):
    exe = tmp_path / "walk_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "long_context_exact_ra_amd", "csrc"),
           os.path.join(HERE, "walk_check.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert " 0 failure(s)" in out and "runtime error" not in out, out
