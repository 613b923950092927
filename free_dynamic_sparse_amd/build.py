"""Build libsolattn.so (the HIP kernels and their C ABI) for gfx950, in-tree.

    python -m free_dynamic_sparse_amd.build [--asm]

Compiles every source under csrc/ with hipcc, one process per file, and
links them into free_dynamic_sparse_amd/_lib/libsolattn.so.  --asm also
keeps the gfx950 assembly under _build/ for inspection.
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(OUT_DIR, "libsolattn.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

# Packed fp32 (v_pk_fma_f32 and friends) stays off: hipcc would otherwise
# form them from plain float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
                "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def _compile(src: str, asm: bool) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON_FLAGS + DEVICE_FLAGS + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if asm:
        cmd += ["--save-temps"]
    proc = subprocess.run(cmd, cwd=BUILD_DIR, capture_output=True, text=True)
    errs = "\n".join(line for line in proc.stderr.splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in line)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if errs.strip():
        sys.stderr.write(errs + "\n")
    return obj


def build(asm: bool = False) -> str:
    """Compile and link libsolattn.so; returns its path."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm), srcs))
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed:\n{proc.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(asm="--asm" in sys.argv[1:]))
