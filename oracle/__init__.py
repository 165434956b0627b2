"""CPU oracle for the MosaicQuant fused W4A4 + sparse-residual path.

TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the benchmark's
CPU-baseline leg are the only users. The HIP library never imports, links or
calls anything here, and this package never imports the library.

This module marshals numpy arrays into ``liboracle.so`` (built from
``oracle.c`` by :func:`build`); every step of the arithmetic is in the C file,
which cites the passages of the MosaicQuant summary it follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fno-strict-aliasing", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(extra_flags=(), out=LIB, src=SRC) -> str:
    """Compile the oracle with gcc (no contraction, no fast-math)."""
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib = None
_libs = {}

_i64 = C.c_int64
_p = C.c_void_p


def load(path: str = LIB):
    """Load (building first if absent) and declare argument types."""
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        if path != LIB:
            raise FileNotFoundError(path)
        build()
    lib = C.CDLL(path)
    lib.or_f32_to_f16_bits.restype = C.c_uint16
    lib.or_f32_to_f16_bits.argtypes = [C.c_float]
    lib.or_f16_bits_to_f32.restype = C.c_float
    lib.or_f16_bits_to_f32.argtypes = [C.c_uint16]
    lib.or_quantize_act.argtypes = [_p, C.c_int, _i64, _i64, _p, _p]
    lib.or_hessian_diag.argtypes = [_p, C.c_int, _i64, _i64, _p]
    lib.or_quantize_weights.argtypes = [_p, _i64, _i64, C.c_int, _p, _p, _p, _p, _p]
    lib.or_delta_scores.argtypes = [_p, _p, _i64, _i64, C.c_int, C.c_int, C.c_int, _p]
    lib.or_select_topk.argtypes = [_p, _i64, _i64, _i64, _p, _p, _p]
    lib.or_pack_weights.argtypes = [_p, _i64, _i64, C.c_int, C.c_int, C.c_int, _p, _p, _i64,
                                    _p, _p, _p]
    lib.or_accumulators.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, C.c_int,
                                    C.c_int, C.c_int, _p, _p]
    lib.or_output.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _p]
    lib.or_distortion.argtypes = [_p, _i64, _p, _p, _i64, _i64, C.c_int, C.c_int, C.c_int, _p,
                                  _p, _p]
    lib.or_smooth_factors.argtypes = [_p, C.c_int, _i64, _i64, _p, _i64, _p, _p]
    lib.or_scale_columns.argtypes = [_p, C.c_int, _i64, _i64, _p, _p]
    for f in ("or_quantize_act", "or_hessian_diag", "or_quantize_weights", "or_delta_scores",
              "or_select_topk", "or_pack_weights", "or_accumulators", "or_output",
              "or_distortion", "or_smooth_factors", "or_scale_columns"):
        getattr(lib, f).restype = C.c_int
    _libs[path] = lib
    return lib


class Oracle:
    """numpy front end over one build of the oracle library."""

    def __init__(self, path: str = LIB):
        self.lib = load(path)

    @staticmethod
    def _ptr(a):
        return None if a is None else a.ctypes.data_as(C.c_void_p)

    def _check(self, rc, what):
        if rc != 0:
            raise ValueError(f"oracle {what} returned {rc}")

    # -- scalar conversions
    def f16_bits(self, f: float) -> int:
        return int(self.lib.or_f32_to_f16_bits(C.c_float(f)))

    def f16_value(self, b: int) -> float:
        return float(self.lib.or_f16_bits_to_f32(C.c_uint16(b)))

    # -- O1
    def quantize_act(self, x: np.ndarray):
        x = np.ascontiguousarray(x)
        dt = 1 if x.dtype == np.uint16 else 0
        if dt == 0:
            x = np.ascontiguousarray(x, dtype=np.float32)
        M, K = x.shape
        xq = np.zeros((M, K // 2), np.uint8)
        sx = np.zeros(M, np.float32)
        self._check(self.lib.or_quantize_act(self._ptr(x), dt, M, K, self._ptr(xq), self._ptr(sx)),
                    "quantize_act")
        return xq, sx

    # -- O0
    def smooth_factors(self, x: np.ndarray, w: np.ndarray):
        """Per-channel migration factors (s, r = 1/s), fp32 [K] each."""
        x = np.ascontiguousarray(x)
        dt = 1 if x.dtype == np.uint16 else 0
        if dt == 0:
            x = np.ascontiguousarray(x, dtype=np.float32)
        w = np.ascontiguousarray(w, dtype=np.float32)
        M, K = x.shape
        N = w.shape[0]
        s = np.zeros(K, np.float32)
        r = np.zeros(K, np.float32)
        self._check(self.lib.or_smooth_factors(self._ptr(x), dt, M, K, self._ptr(w), N, self._ptr(s),
                                               self._ptr(r)), "smooth_factors")
        return s, r

    def scale_columns(self, a: np.ndarray, c: np.ndarray) -> np.ndarray:
        """fp32(a[i][k] * c[k]) for an fp32 or bf16-bits (uint16) matrix."""
        a = np.ascontiguousarray(a)
        dt = 1 if a.dtype == np.uint16 else 0
        if dt == 0:
            a = np.ascontiguousarray(a, dtype=np.float32)
        R, K = a.shape
        out = np.zeros((R, K), np.float32)
        self._check(self.lib.or_scale_columns(self._ptr(a), dt, R, K,
                                              self._ptr(np.ascontiguousarray(c, dtype=np.float32)),
                                              self._ptr(out)), "scale_columns")
        return out

    def migrate(self, x_raw: np.ndarray, w: np.ndarray):
        """The migrated layer (X^, W^) in fp32, and (s, r)."""
        s, r = self.smooth_factors(x_raw, w)
        return self.scale_columns(x_raw, r), self.scale_columns(w, s), s, r

    # -- O4
    def hessian_diag(self, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x)
        dt = 1 if x.dtype == np.uint16 else 0
        if dt == 0:
            x = np.ascontiguousarray(x, dtype=np.float32)
        M, K = x.shape
        h = np.zeros(K, np.float32)
        self._check(self.lib.or_hessian_diag(self._ptr(x), dt, M, K, self._ptr(h)), "hessian")
        return h

    # -- O2/O3 unpacked view
    def quantize_weights(self, w: np.ndarray, group: int = 128):
        w = np.ascontiguousarray(w, dtype=np.float32)
        N, K = w.shape
        q = np.zeros((N, K), np.int8)
        r = np.zeros((N, K), np.int8)
        e = np.zeros((N, K), np.float32)
        ep = np.zeros((N, K), np.float32)
        sw = np.zeros((N, K // group), np.uint16)
        self._check(self.lib.or_quantize_weights(self._ptr(w), N, K, group, self._ptr(q),
                                                 self._ptr(sw), self._ptr(r), self._ptr(e),
                                                 self._ptr(ep)), "quantize_weights")
        return dict(q=q, r=r, e=e, ep=ep, sw=sw)

    # -- O5
    def delta_scores(self, w, h, group=128, bn=64, bk=64) -> np.ndarray:
        w = np.ascontiguousarray(w, dtype=np.float32)
        h = np.ascontiguousarray(h, dtype=np.float32)
        N, K = w.shape
        d = np.zeros((N // bn) * (K // bk), np.float64)
        self._check(self.lib.or_delta_scores(self._ptr(w), self._ptr(h), N, K, group, bn, bk,
                                             self._ptr(d)), "delta_scores")
        return d

    # -- O6
    def select_topk(self, delta, nbr, nbc, k_blocks):
        delta = np.ascontiguousarray(delta, dtype=np.float64)
        row_ptr = np.zeros(nbr + 1, np.int32)
        col_idx = np.zeros(max(k_blocks, 1), np.int32)
        sel = np.zeros(nbr * nbc, np.uint8)
        self._check(self.lib.or_select_topk(self._ptr(delta), nbr, nbc, k_blocks,
                                            self._ptr(row_ptr), self._ptr(col_idx),
                                            self._ptr(sel)), "select_topk")
        return row_ptr, col_idx[:k_blocks].copy(), sel

    def select_blocks(self, w, h, k_blocks, group=128, bn=64, bk=64):
        N, K = w.shape
        d = self.delta_scores(w, h, group, bn, bk)
        row_ptr, col_idx, sel = self.select_topk(d, N // bn, K // bk, k_blocks)
        return row_ptr, col_idx, d, sel

    # -- O7
    def pack_weights(self, w, row_ptr, col_idx, group=128, bn=64, bk=64):
        w = np.ascontiguousarray(w, dtype=np.float32)
        N, K = w.shape
        nnz = int(len(col_idx))
        wq = np.zeros((N, K // 2), np.uint8)
        sw = np.zeros((N, K // group), np.uint16)
        rq = np.zeros((max(nnz, 1), bn, bk // 2), np.uint8)
        row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
        col_idx = np.ascontiguousarray(col_idx, dtype=np.int32)
        self._check(self.lib.or_pack_weights(self._ptr(w), N, K, group, bn, bk,
                                             self._ptr(row_ptr), self._ptr(col_idx), nnz,
                                             self._ptr(wq), self._ptr(sw), self._ptr(rq)),
                    "pack_weights")
        return wq, sw, rq[:nnz].copy()

    # -- O8
    def accumulators(self, xq, wq, row_ptr, col_idx, rq, K, group=128, bn=64, bk=64):
        M, N = xq.shape[0], wq.shape[0]
        G = K // group
        nnz = int(len(col_idx))
        P = np.zeros((M, N, G), np.int32)
        Pr = np.zeros((M, N, G), np.int32)
        rq_c = np.ascontiguousarray(rq if nnz else np.zeros((1, bn, bk // 2), np.uint8))
        col_c = np.ascontiguousarray(col_idx if nnz else np.zeros(1, np.int32), dtype=np.int32)
        self._check(self.lib.or_accumulators(
            self._ptr(np.ascontiguousarray(xq)), self._ptr(np.ascontiguousarray(wq)),
            self._ptr(np.ascontiguousarray(row_ptr, dtype=np.int32)), self._ptr(col_c),
            self._ptr(rq_c), nnz, M, N, K, group, bn, bk, self._ptr(P), self._ptr(Pr)),
            "accumulators")
        return P, Pr

    # -- O9
    def output(self, sx, sw, P, Pr) -> np.ndarray:
        M, N, G = P.shape
        y = np.zeros((M, N), np.float64)
        self._check(self.lib.or_output(self._ptr(np.ascontiguousarray(sx, dtype=np.float32)),
                                       self._ptr(np.ascontiguousarray(sw, dtype=np.uint16)),
                                       self._ptr(np.ascontiguousarray(P)),
                                       self._ptr(np.ascontiguousarray(Pr)), M, N, G,
                                       self._ptr(y)), "output")
        return y

    # -- O10
    def distortion(self, x, w, h, mask, group=128, bn=64, bk=64):
        x = np.ascontiguousarray(x, dtype=np.float32)
        w = np.ascontiguousarray(w, dtype=np.float32)
        h = np.ascontiguousarray(h, dtype=np.float32)
        mask = np.ascontiguousarray(mask, dtype=np.uint8)
        M, K = x.shape
        N = w.shape[0]
        de = C.c_double()
        dd = C.c_double()
        self._check(self.lib.or_distortion(self._ptr(x), M, self._ptr(w), self._ptr(h), N, K,
                                           group, bn, bk, self._ptr(mask), C.byref(de),
                                           C.byref(dd)), "distortion")
        return de.value, dd.value

    # -- the whole path, as one call chain (used for the CPU baseline and smoke check)
    def forward(self, x_raw, w, k_blocks, group=128, bn=64, bk=64):
        h = self.hessian_diag(x_raw)
        row_ptr, col_idx, delta, _ = self.select_blocks(w, h, k_blocks, group, bn, bk)
        wq, sw, rq = self.pack_weights(w, row_ptr, col_idx, group, bn, bk)
        xq, sx = self.quantize_act(x_raw)
        P, Pr = self.accumulators(xq, wq, row_ptr, col_idx, rq, w.shape[1], group, bn, bk)
        y = self.output(sx, sw, P, Pr)
        return dict(h=h, row_ptr=row_ptr, col_idx=col_idx, delta=delta, wq=wq, sw=sw, rq=rq,
                    xq=xq, sx=sx, P=P, Pr=Pr, y=y)
