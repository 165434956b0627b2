"""Host checks of arithmetic shortcuts the HIP kernels rely on, emulated in C
(tests/host_arith.c) and compared with the plain definitions:

* the GEMM's division-free fp32(s / 14) for the residual grid equals the
  correctly rounded quotient for every finite fp16 group scale;
* the quantizers' division-free code (a product by the reciprocal, the exact
  division only near a rounding boundary) equals rint(v / s), ties to even, on
  random scales and values, half of them on or next to a half-integer quotient.
"""
import ctypes as C
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def arith(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("arith") / "libhost_arith.so")
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
                    "-o", out, os.path.join(HERE, "host_arith.c"), "-lm"], check=True)
    lib = C.CDLL(out)
    lib.div14_mismatches.restype = C.c_long
    lib.rint_quot_mismatches.restype = C.c_long
    lib.rint_quot_mismatches.argtypes = [C.c_uint64, C.c_long]
    return lib


def test_division_free_residual_scale_is_exact(arith):
    assert arith.div14_mismatches() == 0


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_division_free_quantizer_code_is_exact(arith, seed):
    assert arith.rint_quot_mismatches(seed, 2_000_000) == 0
