"""Build libtwomamba.so in-tree with hipcc for gfx950.

Usage: ``python -m second_order_ssm_amd.build`` (or ``build()`` from Python).
Each source compiles to an object under ``second_order_ssm_amd/_build`` in
parallel, then everything links into ``second_order_ssm_amd/libtwomamba.so``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtwomamba.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include")]
# Packed-fp32 VALU ops are switched off for all device code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Per-source extra device flags.  The 2Mamba-E kernel's row maxima are plain
# fmaxf chains over MFMA results, and the 2Mamba kernels' lane maxima of |q|,
# |k|, |v|; without NaN semantics the compiler emits v_max3 directly instead of
# canonicalising every operand first (NaN inputs are undefined for the operator).
FILE_FLAGS = {"exp_mfma.hip": ["-fno-honor-nans"], "sq_mfma.hip": ["-fno-honor-nans"]}


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, src + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, *COMMON, *DEVICE, *FILE_FLAGS.get(src, []), "-x", "hip", "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, "-x", "c++", "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(8, len(srcs))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


SANITIZED_LIB = os.path.join(OBJ, "libtwomamba_hostsan.so")


def build_host_sanitized(verbose: bool = False) -> str:
    """Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the C ABI
    (argument validation, path choice, workspace layout: csrc/api.cpp), compiled
    by g++ and linked with the library's unchanged HIP objects.  Device code is
    not instrumented.  Load it with gcc's libasan preloaded (see
    tests/test_abi_sanitized.py); returns its path."""
    if not all(os.path.exists(os.path.join(OBJ, f + ".o")) for f in sources()):
        build(verbose)
    gxx = shutil.which("g++") or "g++"
    api_o = os.path.join(OBJ, "api_hostsan.o")
    cmd = [gxx, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-std=c++17", "-fPIC",
           "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, "api.cpp"), "-o", api_o]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized compile failed\n{r.stdout}\n{r.stderr}")
    objs = [os.path.join(OBJ, f + ".o") for f in sources() if f != "api.cpp"]
    tmp = SANITIZED_LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", api_o, *objs, "-o", tmp, "-lasan", "-lubsan"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SANITIZED_LIB)
    return SANITIZED_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
