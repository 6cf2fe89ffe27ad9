"""Build libpa.so for gfx950 in-tree.

    python paged_kv_cache_238_amd/build.py

Every csrc/*.hip is compiled in two passes, in parallel across sources:

1. the device pass (gfx950 code object bundle), built without packed-fp32
   instructions (the target feature is switched off for this pass only; the
   host compiler does not know the feature);
2. the host pass, which embeds that bundle (clang's
   -fcuda-include-gpubinary, the step the HIP driver otherwise runs
   internally).

The objects are then linked into one shared library next to this file.
Intermediate files go to _build/ at the repository root.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpa.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["pa_api.hip", "decode.hip", "decode_mfma.hip", "decode_prefix.hip", "merge.hip",
           "write_kv.hip", "copy_blocks.hip"]
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")
DEVICE_ONLY_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def clang() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    for cand in (os.environ.get("PA_CLANG"), os.path.join(rocm, "lib/llvm/bin/clang++"),
                 os.path.join(rocm, "llvm/bin/clang++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("ROCm clang++ not found (ROCm is required to build libpa.so)")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


def _common(extra: list[str] | None) -> list[str]:
    return ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Wall", "-Wno-unused-function",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC, *(extra or [])]


def commands(src: str, extra: list[str] | None = None,
             build_dir: str = BUILD_DIR) -> list[list[str]]:
    """Device pass, then host pass, for one source file."""
    stem = os.path.join(build_dir, os.path.splitext(src)[0])
    path = os.path.join(CSRC, src)
    dev = [clang(), *_common(extra), "--offload-device-only", *DEVICE_ONLY_FLAGS,
           "-c", path, "-o", stem + ".hipfb"]
    host = [clang(), *_common(extra), "--offload-host-only", "-c", path,
            "-Xclang", "-fcuda-include-gpubinary", "-Xclang", stem + ".hipfb",
            "-o", stem + ".o"]
    return [dev, host]


def link_command(out: str, build_dir: str = BUILD_DIR) -> list[str]:
    objs = [os.path.join(build_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]


def _run(cmd: list[str], verbose: bool) -> str:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"{os.path.basename(cmd[0])} failed with status "
                           f"{res.returncode}:\n{res.stdout}{res.stderr}")
    return res.stdout + res.stderr


def build(verbose: bool = False, extra: list[str] | None = None, out: str = LIB,
          build_dir: str = BUILD_DIR) -> str:
    """Compile and link; `extra` compiler flags, `out` library path and
    `build_dir` for intermediates (defaults: libpa.so next to this file,
    _build/)."""
    os.makedirs(build_dir, exist_ok=True)

    def one(src: str) -> str:
        return "".join(_run(c, verbose) for c in commands(src, extra, build_dir))

    workers = max(1, min(len(SOURCES), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        logs = list(ex.map(one, SOURCES))
    for log in logs:
        if log.strip():
            sys.stderr.write(log)
    tmp = out + ".tmp"
    _run(link_command(tmp, build_dir), verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build libpa.so (gfx950)")
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("-D", "--define", action="append", default=[], metavar="NAME=VALUE",
                    help="extra preprocessor definition (a build variant, e.g. PA_V_SWIZZLE=0)")
    ap.add_argument("--out", default=LIB, help="library path (default: the package's libpa.so)")
    a = ap.parse_args()
    bdir = BUILD_DIR if not a.define else os.path.join(
        BUILD_DIR, "variant_" + "_".join(d.replace("=", "") for d in a.define))
    print(build(verbose=a.verbose, extra=[f"-D{d}" for d in a.define], out=os.path.abspath(a.out),
                build_dir=bdir))
