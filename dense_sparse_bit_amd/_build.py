"""Build libmq.so (the HIP library) in-tree with hipcc for gfx950.

    python dense_sparse_bit_amd/_build.py

A standalone script (it imports nothing from the package, whose import needs the
built library). Cross-compiles without a GPU. Objects go to
dense_sparse_bit_amd/_build/, the shared library to dense_sparse_bit_amd/libmq.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    # packed fp32 instructions stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE behaviour the bit-exact steps rely on
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-fno-fast-math",
]
# per-source extra flags: the preparation kernels must not contract a*b+c
SOURCES = {
    "prep.hip": ["-ffp-contract=off"],
    "gemm.hip": [],
    "api.hip": ["-ffp-contract=off"],
}


def _compile(name: str, flags: list) -> str:
    src = os.path.join(CSRC, name)
    out = os.path.join(OBJ, name.replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON, *flags, "-c", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {name}:\n{r.stderr}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), SOURCES.items()))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
