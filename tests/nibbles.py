"""Test-side helpers: decode the packed int4 formats with numpy.

Written independently of both the oracle's C code and the HIP library, so a
mistake in either one's nibble order or sign handling shows up as a mismatch.
Format: two's-complement int4, low nibble holds the even index. The oracle
returns row-major arrays; the library's packed layouts (described in
include/mq.h) are converted back to row-major here with reshapes and transposes
only, so the comparison is element by element.
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
    """group-major [K/128][M][64] bytes -> [M][K/2]"""
    a = np.asarray(dev, np.uint8).reshape(K // 128, M, 64)
    return a.transpose(1, 0, 2).reshape(M, K // 2)


def wq_to_rowmajor(dev: np.ndarray, N: int, K: int) -> np.ndarray:
    """tiles [N/16][G][kc 4][row 16][16 B] -> [N][K/2]"""
    G = K // 128
    a = np.asarray(dev, np.uint8).reshape(N // 16, G, 4, 16, 16)
    return a.transpose(0, 3, 1, 2, 4).reshape(N, K // 2)


def sw_to_rowmajor(dev: np.ndarray, N: int, K: int):
    """[N/16][G4][row 16][4] u16 -> ([N][G] scales, [N][4*G4 - G] padding slots)"""
    G = K // 128
    G4 = (G + 3) // 4
    a = np.asarray(dev).view(np.uint16).reshape(N // 16, G4, 16, 4)
    full = a.transpose(0, 2, 1, 3).reshape(N, 4 * G4)
    return full[:, :G], full[:, G:]
