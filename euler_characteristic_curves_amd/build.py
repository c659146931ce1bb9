"""Build libecc_mi355.so in-tree with hipcc for gfx950.

Usage: ``python -m euler_characteristic_curves_amd.build`` (also called by
``__graft_entry__.build()``).  Sources are compiled in parallel into
``_build/`` at the repository root and linked into
``euler_characteristic_curves_amd/libecc_mi355.so``.  The benchmark's
sigmoid-rate probe is linked on its own into ``libecc_sigmoid_rate.so``.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libecc_mi355.so")

SOURCES = ["ecc_api.cpp", "ecc_hard.hip", "ecc_soft.hip", "ecc_soft_grad.hip", "ecc_height.hip", "ecc_static.hip"]
RATE_SOURCE = "ecc_sigmoid_rate.hip"
RATE_LIB = os.path.join(PKG, "libecc_sigmoid_rate.so")
ARCH = os.environ.get("ECC_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libecc_mi355)")


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc()] + COMMON + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False):
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        results = list(ex.map(_compile, SOURCES + [RATE_SOURCE]))
    rate_obj = results.pop()[0]
    objs = [o for o, _ in results]
    if verbose:
        for _, err in results:
            if err.strip():
                print(err, file=sys.stderr)
    for lib, lib_objs in ((LIB, objs), (RATE_LIB, [rate_obj])):
        tmp = lib + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + lib_objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
