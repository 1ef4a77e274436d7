"""The LDS layouts read both as rows and transposed (the backward's tiles,
the feedforward GEMM's W stage) and the GEMM's X pair stage
(``csrc/ra_lds.h``) checked on the host:
every lane of every operand read receives the tile elements the MFMA
operand layout asks for, the DMA lands every row and granule where the
readers look, and every read touches each LDS bank once per cycle (the
unswizzled layout is shown to fail that).  Built with g++ under
AddressSanitizer and UBSan."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_lds_layouts(tmp_path):
    exe = str(tmp_path / "lds_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "long_context_exact_ra_amd", "csrc"),
           os.path.join(ROOT, "tests", "lds_check.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failure(s)" in r.stdout
