"""Build the HIP library ``libpa.so`` in-tree for gfx950, and beside it
``libpa_stream.so``, the benchmark's bandwidth reference kernels (a plain
streaming read and copy; not part of the library's C ABI).

    python -m paged_kv_cache_pa_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libpa.so")
SOURCES = ["pa_kernels.hip", "pa_abi.cpp", "block_manager.cpp"]
STREAM_LIB_PATH = os.path.join(PKG, "libpa_stream.so")
STREAM_SOURCES = ["stream_ref.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build(verbose: bool = False) -> str:
    """Both libraries; returns the path of libpa.so."""
    _build_one(SOURCES, LIB_PATH, verbose)
    _build_one(STREAM_SOURCES, STREAM_LIB_PATH, verbose)
    return LIB_PATH


def _build_one(sources, lib_path, verbose):
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-shared",
           # packed fp32 VALU ops stay off (no v_pk_*_f32 anywhere in this library)
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    cmd += [os.path.join(CSRC, s) for s in sources]
    cmd += ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, lib_path)


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
