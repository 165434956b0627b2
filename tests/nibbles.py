"""Test-side helpers: decode the packed int4 formats with numpy.

Written independently of both the oracle's C code and the HIP library, so a
mistake in either one's nibble order or sign handling shows up as a mismatch.
The oracle packs two's-complement int4 codes, low nibble = even index, in
row-major arrays. The library packs the same codes in its own word encoding
(include/mq.h: per 32-bit word of 8 consecutive codes, nibble e holds |c_e| in
its low three bits and the sign of code (e - 1) mod 8 in its high bit) and in
tiled layouts. The converters below undo the layouts with reshapes and
transposes only and the word encoding with a decoder written from that
definition; the decoder also re-encodes and insists on the same bytes, so an
invalid word (a negative zero, a stray bit) fails the comparison.
"""
import numpy as np


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """uint8 [..., K/2] -> int8 [..., K]"""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0x0F).astype(np.int8)
    hi = (p >> 4).astype(np.int8)
    lo = np.where(lo >= 8, lo - 16, lo).astype(np.int8)
    hi = np.where(hi >= 8, hi - 16, hi).astype(np.int8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """int [..., K] (values in [-8, 7]) -> two's-complement nibbles uint8 [..., K/2]"""
    c = np.asarray(codes).astype(np.int64) & 15
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def lib_codes(packed: np.ndarray) -> np.ndarray:
    """library word encoding, uint8 [..., 4W] -> int8 codes [..., 8W]"""
    p = np.asarray(packed, dtype=np.uint8)
    assert p.shape[-1] % 4 == 0
    nib = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    nib[..., 0::2] = p & 0x0F
    nib[..., 1::2] = p >> 4
    mag = (nib & 7).astype(np.int8)
    top = (nib >> 3).reshape(nib.shape[:-1] + (-1, 8))
    # the high bit of nibble e is the sign of code e - 1: code c's sign sits in nibble c + 1
    sign = np.roll(top, -1, axis=-1).reshape(nib.shape)
    codes = np.where(sign == 1, -mag, mag).astype(np.int8)
    again = lib_pack(codes)
    if not np.array_equal(again, p):
        bad = np.argwhere(again != p)[0]
        raise AssertionError(f"invalid library code word at byte {tuple(bad)}: {p[tuple(bad)]:#04x}")
    return codes


def lib_pack(codes: np.ndarray) -> np.ndarray:
    """int codes [..., 8W] in [-7, 7] -> library word encoding uint8 [..., 4W]"""
    c = np.asarray(codes).astype(np.int64)
    assert c.shape[-1] % 8 == 0 and np.all(np.abs(c) <= 7)
    mag = np.abs(c)
    neg = (c < 0).astype(np.int64).reshape(c.shape[:-1] + (-1, 8))
    top = np.roll(neg, 1, axis=-1).reshape(c.shape)     # nibble e carries the sign of code e - 1
    nib = mag | (top << 3)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def lib_to_twos(packed: np.ndarray) -> np.ndarray:
    """library word encoding -> the oracle's two's-complement nibble bytes (same shape)"""
    return pack_int4(lib_codes(packed))


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def f32_to_f16_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def residual_dense(rq, row_ptr, col_idx, N, K, bn, bk) -> np.ndarray:
    """Scatter the CSR residual payload into a dense int8 [N][K] code matrix."""
    R = np.zeros((N, K), np.int8)
    rows = unpack_int4(rq) if len(col_idx) else np.zeros((0, bn, bk), np.int8)
    for i in range(N // bn):
        for p in range(row_ptr[i], row_ptr[i + 1]):
            j = col_idx[p]
            R[i * bn:(i + 1) * bn, j * bk:(j + 1) * bk] = rows[p]
    return R


def rel_err(y, y_ref) -> float:
    """max over (m, n) of |y - ref| / max(|ref|, 0.1 * rms(ref[m, :]))"""
    y = np.asarray(y, np.float64)
    ref = np.asarray(y_ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    den = np.maximum(np.abs(ref), 0.1 * rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(y - ref) / den)) if y.size else 0.0


# ---- the library's packed layouts -> row-major -----------------------------
def xq_to_rowmajor(dev: np.ndarray, M: int, K: int) -> np.ndarray:
    """group-major [K/128][M][64] library bytes -> [M][K/2] two's-complement nibbles"""
    a = np.asarray(dev, np.uint8).reshape(K // 128, M, 64)
    return lib_to_twos(a.transpose(1, 0, 2).reshape(M, K // 2))


def wq_to_rowmajor(dev: np.ndarray, N: int, K: int) -> np.ndarray:
    """tiles [N/16][G][kc 4][row 16][16 B] library bytes -> [N][K/2] two's-complement nibbles"""
    G = K // 128
    a = np.asarray(dev, np.uint8).reshape(N // 16, G, 4, 16, 16)
    return lib_to_twos(a.transpose(0, 3, 1, 2, 4).reshape(N, K // 2))


def rq_to_twos(dev: np.ndarray) -> np.ndarray:
    """residual payload [nnz][bn][32] library bytes -> two's-complement nibbles"""
    a = np.asarray(dev, np.uint8)
    return lib_to_twos(a) if a.size else a.copy()


def sw_to_rowmajor(dev: np.ndarray, N: int, K: int):
    """[N/16][G4][row 16][4] u16 -> ([N][G] scales, [N][4*G4 - G] padding slots)"""
    G = K // 128
    G4 = (G + 3) // 4
    a = np.asarray(dev).view(np.uint16).reshape(N // 16, G4, 16, 4)
    full = a.transpose(0, 2, 1, 3).reshape(N, 4 * G4)
    return full[:, :G], full[:, G:]
