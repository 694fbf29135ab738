"""Builds libstatekv.so (HIP kernels + C ABI) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
LIB_NAME = "libstatekv.so"
SOURCES = ["statekv_kernels.hip", "statekv_runtime.hip"]


def library_path() -> str:
    return os.path.join(PKG_DIR, LIB_NAME)


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the StateKV HIP library cannot be built")


def compile_command(out: str) -> list:
    return [
        _hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-mcode-object-version=5",
        # Packed fp32 instructions are kept out of every kernel.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # Matrix-core results in ordinary vector registers: the softmax and
        # score arithmetic reads them directly instead of copying them out of
        # accumulation registers first (score pass 3-6 % faster on the long
        # pools, the text-phase kernel 5 %).
        "-mllvm", "--amdgpu-mfma-vgpr-form",
        "-I", INCLUDE, "-I", CSRC,
        # Every symbol resolved at link time: a declaration without its
        # definition fails the build instead of the first load.
        "-Wl,-z,defs",
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Compile the library (always) and return its path."""
    out = library_path()
    tmp = out + ".tmp"
    proc = subprocess.run(compile_command(tmp), capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + proc.stdout + proc.stderr)
    if verbose and proc.stderr:
        print(proc.stderr)
    os.replace(tmp, out)
    return out
