"""Build libpa.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m prefill_block_table_amd.build

Always recompiles.  The library lands next to this file so it travels with
the source tree; nothing is installed anywhere else.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libpa.so")
SOURCES = ["pa_api.cpp", "kv_write.hip", "decode.hip", "prefill.hip", "input_prep.hip", "gemv.hip"]

# Packed fp32 VALU ops are switched off for all device code.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", "-Werror=uninitialized"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa)")


def _git_rev() -> str:
    try:
        out = subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=HERE,
                             capture_output=True, text=True, timeout=10)
        rev = out.stdout.strip() or "unknown"
        dirty = subprocess.run(["git", "status", "--porcelain", "--", "."], cwd=HERE,
                               capture_output=True, text=True, timeout=10).stdout.strip()
        return rev + ("+dirty" if dirty else "")
    except Exception:
        return "unknown"


def build(extra_flags=(), out_path: str = LIB_PATH, verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out_path + ".tmp"
    cmd = [_hipcc(), *HIP_FLAGS, f'-DPA_GIT_REV="{_git_rev()}"', *extra_flags,
           "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
