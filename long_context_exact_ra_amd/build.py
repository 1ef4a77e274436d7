"""Build the C-ABI shared library ``libra_attn.so`` in-tree for gfx950.

The HIP kernels are compiled with hipcc for ``--offload-arch=gfx950``; the
host-side C ABI (validation, planner, errors) is plain C++ built with g++.
Packed-FP32 VALU instructions are disabled for all device code.
"""

from __future__ import annotations

import hashlib
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libra_attn.so")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
# Per-source additions.  The forward kernels take finite inputs (the C ABI
# says so), so their row maxima need no NaN quieting before v_max3.
FILE_FLAGS = {"blockwise_fwd.hip": ["-fno-honor-nans"]}
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Werror",
             "-I", INCLUDE, "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def _flags_key() -> bytes:
    """The compile flags that shape the code, without include paths (which
    differ between machines)."""
    flags = [f for f in HIP_FLAGS if not f.startswith("/") and f != "-I"]
    return repr((flags, sorted(FILE_FLAGS.items()))).encode()


def device_sources_sha16() -> str:
    """First 16 hex digits of the SHA-256 over the device compile flags and
    sources (the .hip files and the headers they include, in name order):
    the build id ``ra_version()`` reports after "+"."""
    h = hashlib.sha256(_flags_key())
    for src in sorted(os.listdir(CSRC)):
        if src.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, src), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


# The sources the forward kernel is compiled from.
FWD_SOURCES = ("blockwise_fwd.hip", "ra_device.h", "ra_internal.h", "ra_walk.h")


def fwd_sources_sha16() -> str:
    """First 16 hex digits of the SHA-256 over the compile flags and the
    forward kernel's sources."""
    h = hashlib.sha256(_flags_key())
    for src in FWD_SOURCES:
        with open(os.path.join(CSRC, src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def build(verbose: bool = True) -> str:
    """Compile every source and link ``libra_attn.so``; returns its path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    cxx = shutil.which("g++") or "g++"
    build_id = f'-DRA_BUILD_ID="{device_sources_sha16()}"'
    objs = []
    for src in sorted(os.listdir(CSRC)):
        path = os.path.join(CSRC, src)
        obj = os.path.join(BUILD, src + ".o")
        if src.endswith(".hip"):
            _run([HIPCC, *HIP_FLAGS, *FILE_FLAGS.get(src, []), "-c", path, "-o", obj], verbose)
        elif src.endswith(".cpp"):
            _run([cxx, *CXX_FLAGS, build_id, "-c", path, "-o", obj], verbose)
        else:
            continue
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
