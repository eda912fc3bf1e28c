"""Build libsparq24.so for gfx950 in-tree with hipcc.

Usage: python -m pruning_quantization_amd.build [-v]

Every call recompiles all sources (objects go to ``_build/`` at the repository
root, the library next to this file).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsparq24.so")

SOURCES = ["api.cpp", "kernels_prune.hip", "kernels_quant.hip", "kernels_energy.hip",
           "kernels_misc.hip", "kernels_operr.hip", "kernels_spgemm.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: no v_pk_*_f32 in any kernel.  No fast-math, no denormal
# flushing: every fp32 step is an IEEE operation.
COMMON = ["-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function", "-fno-fast-math", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    return obj


CHECK_SRC = "check_converts.hip"
CHECK_BIN = os.path.join(PKG, "check_converts")


def _build_check(verbose: bool) -> None:
    """Stand-alone program that checks gfx950's fp8/fp4 conversion instructions
    against the exact encoders over every finite fp32 (run by a GPU test)."""
    cmd = [HIPCC, *COMMON, os.path.join(CSRC, CHECK_SRC), "-o", CHECK_BIN + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for check_converts:\n" + r.stdout + r.stderr)
    shutil.move(CHECK_BIN + ".tmp", CHECK_BIN)


def build(verbose: bool = False) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES) + 1, os.cpu_count() or 4)) as ex:
        chk = ex.submit(_build_check, verbose)
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
        chk.result()
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    shutil.move(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
