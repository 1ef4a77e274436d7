"""The host side of the C ABI (csrc/ra_host.cpp) built with g++
AddressSanitizer and UndefinedBehaviorSanitizer and driven by
host_sanitize_driver.cpp (stub launchers, fake device pointers): the
planner at every workload's shape, validation, the key-split and workspace
helpers, and the derived grid sizes.  CPU only; the device code is not
built here."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_code_under_sanitizers(tmp_path):
    exe = tmp_path / "host_driver"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "long_context_exact_ra_amd", "csrc"),
           os.path.join(ROOT, "long_context_exact_ra_amd", "csrc", "ra_host.cpp"),
           os.path.join(HERE, "host_sanitize_driver.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
    assert "ok: 0 failure(s)" in out, out
