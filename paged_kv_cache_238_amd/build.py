"""Build libpa.so for gfx950 in-tree with hipcc.

    python paged_kv_cache_238_amd/build.py

Compiles every csrc/*.hip into one shared library next to this file.  All
device code is built without packed-fp32 instructions.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpa.so")
SOURCES = ["pa_api.hip", "decode.hip", "decode_mfma.hip", "decode_prefix.hip", "merge.hip",
           "write_kv.hip", "copy_blocks.hip"]
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


def command(out: str = LIB, extra: list[str] | None = None) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Wall", "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        *(extra or []),
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
