"""Compile the HIP sources of this package into ``libfa.so`` (gfx950 only).

Run ``python io_aware_softmax_attn_amd/build.py`` or call :func:`build_library`
from a module loaded on its own (importing the package first would load the
library that is about to be replaced).
The library is written next to this file, in-tree, through a temporary name and
an atomic rename, so a half-written file is never loaded.
"""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")
SOURCES = ["fa_fwd.hip", "fa_unfused.hip", "fa_decode.hip", "fa_bwd.hip", "fa_api.cpp", "fa_select.cpp"]
HEADERS = [os.path.join(CSRC, "fa_internal.h"), os.path.join(os.path.dirname(PKG_DIR), "include", "fa.h")]
ARCH = "gfx950"
HASH_PATH = LIB_PATH + ".srchash"  # sha256 of the sources and flags libfa.so was built from


def source_hash() -> str:
    """sha256 over the compile flags and the bytes of every source and header."""
    h = hashlib.sha256(" ".join(FLAGS).encode())
    for path in [os.path.join(CSRC, s) for s in SOURCES] + HEADERS:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()


def check_built() -> None:
    """Raise unless libfa.so exists and was built from the current sources."""
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing")
    recorded = None
    if os.path.exists(HASH_PATH):
        with open(HASH_PATH) as f:
            recorded = f.read().strip()
    if recorded != source_hash():
        raise RuntimeError(f"{LIB_PATH} was built from other sources than the current ones; rebuild it with "
                           f"'python io_aware_softmax_attn_amd/build.py'")


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libfa.so")
    return path


FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU ops are kept out of generated code on this part
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def compile_command(out: str) -> list[str]:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    return [hipcc(), *FLAGS, *srcs, "-o", out]


def build_library(verbose: bool = False) -> str:
    hipcc()
    digest = source_hash()
    fd, tmp = tempfile.mkstemp(prefix="libfa.", suffix=".so.tmp", dir=PKG_DIR)
    os.close(fd)
    try:
        cmd = compile_command(tmp)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if verbose or res.returncode != 0:
            sys.stderr.write(res.stderr)
        if res.returncode != 0:
            raise RuntimeError(f"building libfa.so failed (exit {res.returncode}): {' '.join(cmd)}")
        os.replace(tmp, LIB_PATH)
        with open(HASH_PATH, "w") as f:
            f.write(digest + "\n")
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
