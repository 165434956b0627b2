"""MI355X (gfx950) MosaicQuant library: Python binding over the C ABI in include/mq.h.

The functions below only marshal torch device tensors (pointers, sizes and the
current HIP stream) into ``libmq.so``; every step of the computation runs in the
library's HIP kernels. There is no CPU fallback: importing this package raises
if the library has not been built (``python dense_sparse_bit_amd/_build.py``),
and every call raises :class:`MQError` on a non-zero status.

Packed tensors use the library's device layouts (include/mq.h): xq is
[K/128][M][64] bytes (group-major), wq is [N/16][K/128][1024] bytes (16-row x
1-group tiles), sw is [N/16][ceil(K/512)][16][4] fp16 bits.
"""
from __future__ import annotations

import ctypes as C
import os

import torch  # loads torch's HIP runtime first, so libmq.so binds to the same one

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmq.so")

MQ_F32, MQ_BF16 = 0, 1
GROUP, BK = 128, 64

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python dense_sparse_bit_amd/_build.py` "
                      "(hipcc, gfx950). There is no fallback implementation.")

_lib = C.CDLL(LIB_PATH)
_p, _i64, _int = C.c_void_p, C.c_int64, C.c_int

_SIGS = {
    "mq_hessian_diag": [_p, _int, _i64, _i64, _p, _p],
    "mq_quantize_act": [_p, _int, _i64, _i64, _p, _p, _p],
    "mq_quantize_act_scaled": [_p, _int, _i64, _i64, _p, _p, _p, _p],
    "mq_hessian_diag_scaled": [_p, _int, _i64, _i64, _p, _p, _p],
    "mq_smooth_factors": [_p, _int, _i64, _i64, _p, _i64, _p, _p, _p],
    "mq_scale_columns": [_p, _i64, _i64, _p, _p, _p],
    "mq_select_blocks": [_p, _p, _i64, _i64, _int, _int, _int, _i64, _p, _p, _p, _p, C.c_size_t, _p],
    "mq_select_blocks_noalloc": [_p, _p, _i64, _i64, _int, _int, _int, _i64, _p, _p, _p, _p],
    "mq_pack_weights": [_p, _i64, _i64, _int, _int, _int, _p, _p, _i64, _p, _p, _p, _p],
    "mq_gemm_w4a4_residual": [_p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _int, _int, _int,
                              _p, _int, _p, _p],
    "mq_gemm_w4a4_dense": [_p, _p, _p, _p, _i64, _i64, _i64, _int, _p, _int, _p, _p],
    "mq_block_map": [_p, _p, _i64, _i64, _i64, _int, _int, _p, _p],
    "mq_read_probe": [_p, _i64, _p, _p],
    "mq_act_one_launch": [_i64, _i64, _i64],
    "mq_gemm_w4a4_residual_act": [_p, _int, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _int, _int, _int,
                                  _p, _p, _p, _int, _p, _int, _p],
    "mq_gemm_w4a4_residual_mapped": [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _int, _int, _int,
                                     _p, _int, _p, _p],
    "mq_gemm_residual_separate": [_p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _int, _int,
                                  _int, _p, _int, _p, _p],
}
for _name, _args in _SIGS.items():
    getattr(_lib, _name).argtypes = _args
    getattr(_lib, _name).restype = C.c_int
_lib.mq_status_string.argtypes = [C.c_int]
_lib.mq_status_string.restype = C.c_char_p
_lib.mq_version.argtypes = []
_lib.mq_version.restype = C.c_int
_lib.mq_select_workspace_bytes.argtypes = [_i64, _i64, _int, _int]
_lib.mq_select_workspace_bytes.restype = C.c_size_t

EXPORTS = tuple(_SIGS) + ("mq_status_string", "mq_version", "mq_select_workspace_bytes")


class MQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


def status_string(status: int) -> str:
    return _lib.mq_status_string(status).decode()


def version() -> int:
    return int(_lib.mq_version())


def lib():
    """The loaded ctypes library (raw C ABI)."""
    return _lib


def _ptr(t):
    if t is None:
        return None
    return C.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _call(fn: str, *args):
    rc = getattr(_lib, fn)(*args)
    if rc != 0:
        raise MQError(fn, rc)


def _x_dtype(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return MQ_F32
    if x.dtype == torch.bfloat16:
        return MQ_BF16
    raise TypeError(f"activations must be float32 or bfloat16, got {x.dtype}")


def _device_contig(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _buf(t, name: str, nbytes: int, dtypes=None, align: int = 1):
    """Checks a caller-supplied buffer before its pointer goes to the library:
    type, dtype, size (at least nbytes), contiguity and alignment. The device is
    checked last, for all operands of a call together (_on_device)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, needs at least {nbytes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if align > 1 and have and t.data_ptr() % align:
        raise ValueError(f"{name} must be {align}-byte aligned")
    return t


def _on_device(**tensors):
    """Every tensor a call hands to the library must live on the GPU."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")


_U8 = (torch.uint8,)
_I32 = (torch.int32,)
_F32 = (torch.float32,)
_SW = (torch.int16, torch.uint16, torch.float16) if hasattr(torch, "uint16") else (torch.int16, torch.float16)


def _shape2(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    return int(t.shape[0]), int(t.shape[1])


# --------------------------------------------------------------------------- a0
def hessian_diag(x: torch.Tensor, out: torch.Tensor | None = None, r: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """h = mean over tokens of x^2 per channel (of x * r when r is given)."""
    M, K = _shape2(x, "x")
    _x_dtype(x)
    _device_contig(x, "x")
    h = torch.empty(K, dtype=torch.float32, device=x.device) if out is None else _buf(out, "h", 4 * K, _F32)
    if r is not None:
        _buf(r, "r", 4 * K, _F32)
    _on_device(x=x, h=h, r=r)
    if r is None:
        _call("mq_hessian_diag", _ptr(x), _x_dtype(x), M, K, _ptr(h), _stream(stream))
    else:
        _call("mq_hessian_diag_scaled", _ptr(x), _x_dtype(x), M, K, _ptr(r), _ptr(h), _stream(stream))
    return h


# --------------------------------------------------------------------------- a4
def quantize_act(x: torch.Tensor, xq: torch.Tensor | None = None, sx: torch.Tensor | None = None,
                 r: torch.Tensor | None = None, stream=None):
    """Returns (xq u8 [K/128][M][64], sx fp32 [M]). With r (fp32 [K], from
    smooth_factors) the migrated activations x * r are quantized."""
    M, K = _shape2(x, "x")
    _x_dtype(x)
    _device_contig(x, "x")
    if xq is None:
        xq = torch.empty((K // GROUP, M, 64), dtype=torch.uint8, device=x.device)
    else:
        _buf(xq, "xq", M * K // 2, _U8, 16)
    if sx is None:
        sx = torch.empty(M, dtype=torch.float32, device=x.device)
    else:
        _buf(sx, "sx", 4 * M, _F32)
    if r is not None:
        _buf(r, "r", 4 * K, _F32, 16)
    _on_device(x=x, xq=xq, sx=sx, r=r)
    if r is None:
        _call("mq_quantize_act", _ptr(x), _x_dtype(x), M, K, _ptr(xq), _ptr(sx), _stream(stream))
    else:
        _call("mq_quantize_act_scaled", _ptr(x), _x_dtype(x), M, K, _ptr(r), _ptr(xq), _ptr(sx),
              _stream(stream))
    return xq, sx


# --------------------------------------------------------------------------- a0' migration
def smooth_factors(x: torch.Tensor, w: torch.Tensor, s=None, r=None, stream=None):
    """Per-channel migration factors (s, r = 1/s), fp32 [K] each (alpha = 1/2)."""
    M, K = _shape2(x, "x")
    N, K2 = _shape2(w, "w")
    if K2 != K:
        raise ValueError(f"x has {K} channels, w has {K2}")
    _x_dtype(x)
    if w.dtype != torch.float32:
        raise TypeError("w must be float32")
    _device_contig(x, "x")
    _device_contig(w, "w")
    s = torch.empty(K, dtype=torch.float32, device=w.device) if s is None else _buf(s, "s", 4 * K, _F32)
    r = torch.empty(K, dtype=torch.float32, device=w.device) if r is None else _buf(r, "r", 4 * K, _F32)
    _on_device(x=x, w=w, s=s, r=r)
    _call("mq_smooth_factors", _ptr(x), _x_dtype(x), M, K, _ptr(w), N, _ptr(s), _ptr(r), _stream(stream))
    return s, r


def scale_columns(w: torch.Tensor, s: torch.Tensor, out=None, stream=None):
    """The migrated weights W diag(s), fp32 [N][K]."""
    N, K = _shape2(w, "w")
    if w.dtype != torch.float32:
        raise TypeError("w must be float32")
    _device_contig(w, "w")
    _buf(s, "s", 4 * K, _F32, 16)
    out = torch.empty_like(w) if out is None else _buf(out, "out", 4 * N * K, _F32, 16)
    _on_device(w=w, s=s, out=out)
    _call("mq_scale_columns", _ptr(w), N, K, _ptr(s), _ptr(out), _stream(stream))
    return out


# --------------------------------------------------------------------------- a2
def select_workspace(N: int, K: int, bn: int = 64, bk: int = BK, device="cuda"):
    """Scratch for select_blocks (per-block ranks, and the scores when they are not
    returned), so the call allocates nothing."""
    n = int(_lib.mq_select_workspace_bytes(N, K, bn, bk))
    return torch.empty(max(n, 8), dtype=torch.uint8, device=device)


def select_blocks(w: torch.Tensor, h: torch.Tensor, k_blocks: int, bn: int = 64, group: int = GROUP,
                  bk: int = BK, out=None, workspace=None, stream=None, return_delta: bool = True):
    """Returns (row_ptr int32 [N/bn+1], col_idx int32 [k_blocks], delta fp64 [NB] or None).
    workspace: optional select_workspace(...) tensor; without it the library takes a
    stream-ordered allocation for the call. return_delta=False passes a NULL score
    output (the scores stay in the scratch)."""
    N, K = _shape2(w, "w")
    if w.dtype != torch.float32 or h.dtype != torch.float32:
        raise TypeError("w and h must be float32")
    _device_contig(w, "w")
    _buf(h, "h", 4 * K, _F32, 16)
    if bn <= 0 or bk <= 0 or N % bn or K % bk:
        raise ValueError(f"blocks {bn}x{bk} do not tile a {N}x{K} layer")
    nb = (N // bn) * (K // bk)
    if not 0 <= k_blocks <= nb:
        raise ValueError(f"k_blocks = {k_blocks} outside [0, {nb}]")
    if out is None:
        row_ptr = torch.empty(N // bn + 1, dtype=torch.int32, device=w.device)
        col_idx = torch.empty(max(k_blocks, 1), dtype=torch.int32, device=w.device)
        delta = torch.empty(max(nb, 1), dtype=torch.float64, device=w.device) if return_delta else None
    else:
        row_ptr, col_idx, delta = out
        _buf(row_ptr, "row_ptr", 4 * (N // bn + 1), _I32)
        _buf(col_idx, "col_idx", 4 * k_blocks, _I32)
        if delta is not None:
            _buf(delta, "delta", 8 * nb, (torch.float64,))
    ws, wsb = None, 0
    if workspace is not None:
        _buf(workspace, "workspace", 0, None, 8)
        ws, wsb = _ptr(workspace), workspace.numel() * workspace.element_size()
    _on_device(w=w, h=h, row_ptr=row_ptr, col_idx=col_idx, delta=delta, workspace=workspace)
    _call("mq_select_blocks", _ptr(w), _ptr(h), N, K, group, bn, bk, k_blocks, _ptr(row_ptr),
          _ptr(col_idx), _ptr(delta), ws, wsb, _stream(stream))
    return row_ptr, col_idx[:k_blocks], (None if delta is None else delta[:nb])


NOALLOC_SCRATCH_BYTES = 4 << 20     # MQ_NOALLOC_SCRATCH_BYTES


def select_blocks_noalloc(w: torch.Tensor, h: torch.Tensor, k_blocks: int, row_ptr: torch.Tensor,
                          col_idx: torch.Tensor, delta: torch.Tensor | None = None, bn: int = 64,
                          group: int = GROUP, bk: int = BK, stream=None):
    """select_blocks into caller-supplied outputs with no allocation at all (the
    library's static scratch): for code under graph capture or in loops that must
    not allocate. delta=None leaves the scores in the scratch. Calls that overlap on
    one GPU race (one scratch array per GPU)."""
    N, K = _shape2(w, "w")
    if w.dtype != torch.float32 or h.dtype != torch.float32:
        raise TypeError("w and h must be float32")
    _device_contig(w, "w")
    _buf(h, "h", 4 * K, _F32, 16)
    if bn <= 0 or bk <= 0 or N % bn or K % bk:
        raise ValueError(f"blocks {bn}x{bk} do not tile a {N}x{K} layer")
    nb = (N // bn) * (K // bk)
    if not 0 <= k_blocks <= nb:
        raise ValueError(f"k_blocks = {k_blocks} outside [0, {nb}]")
    _buf(row_ptr, "row_ptr", 4 * (N // bn + 1), _I32)
    _buf(col_idx, "col_idx", 4 * k_blocks, _I32)
    if delta is not None:
        _buf(delta, "delta", 8 * nb, (torch.float64,))
    _on_device(w=w, h=h, row_ptr=row_ptr, col_idx=col_idx, delta=delta)
    _call("mq_select_blocks_noalloc", _ptr(w), _ptr(h), N, K, group, bn, bk, k_blocks, _ptr(row_ptr),
          _ptr(col_idx), _ptr(delta), _stream(stream))
    return row_ptr, col_idx[:k_blocks], (None if delta is None else delta[:nb])


# --------------------------------------------------------------------------- a1 + a3
def _csr_checks(row_ptr, col_idx, N, bn):
    _buf(row_ptr, "row_ptr", 4 * (N // bn + 1), _I32)
    if col_idx.numel():
        _buf(col_idx, "col_idx", 4 * col_idx.numel(), _I32)
    return int(col_idx.numel())


def pack_weights(w: torch.Tensor, row_ptr: torch.Tensor, col_idx: torch.Tensor, bn: int = 64,
                 group: int = GROUP, bk: int = BK, out=None, stream=None):
    """Returns (wq u8 [N/16][G][1024], sw fp16-bits int16 [N/16][G4][16][4],
    rq u8 [nnz][bn][bk/2]) with G = K/128, G4 = ceil(G/4)."""
    N, K = _shape2(w, "w")
    if w.dtype != torch.float32:
        raise TypeError("w must be float32")
    _device_contig(w, "w")
    nnz = _csr_checks(row_ptr, col_idx, N, bn)
    G = K // group
    if out is None:
        wq = torch.empty((N // 16, G, 1024), dtype=torch.uint8, device=w.device)
        sw = torch.empty((N // 16, (G + 3) // 4, 16, 4), dtype=torch.int16, device=w.device)
        rq = torch.empty((max(nnz, 1), bn, bk // 2), dtype=torch.uint8, device=w.device)
    else:
        wq, sw, rq = out
        _buf(wq, "wq", N * K // 2, _U8, 16)
        _buf(sw, "sw", 8 * N * ((G + 3) // 4), _SW, 8)
        _buf(rq, "rq", nnz * bn * bk // 2, _U8, 16)
    _on_device(w=w, row_ptr=row_ptr, col_idx=col_idx, wq=wq, sw=sw, rq=rq)
    _call("mq_pack_weights", _ptr(w), N, K, group, bn, bk, _ptr(row_ptr),
          _ptr(col_idx) if nnz else None, nnz, _ptr(wq), _ptr(sw), _ptr(rq) if nnz else None,
          _stream(stream))
    return wq, sw, rq[:nnz]


# --------------------------------------------------------------------------- a5..a10
def _y_dtype(dtype) -> int:
    if dtype == torch.float32:
        return MQ_F32
    if dtype == torch.bfloat16:
        return MQ_BF16
    raise TypeError(f"output must be float32 or bfloat16, got {dtype}")


def _gemm_operands(xq, sx, wq, sw, K: int):
    """(M, N) of a GEMM call, after checking the packed operands: M tokens from sx,
    N outputs from the packed weight bytes."""
    if K <= 0 or K % GROUP:
        raise ValueError(f"K = {K} must be a positive multiple of {GROUP}")
    _buf(sx, "sx", 0, _F32)
    M = int(sx.numel())
    if wq.numel() * 2 % K:
        raise ValueError(f"wq holds {wq.numel()} bytes, not a multiple of K/2 = {K // 2}")
    N = int(wq.numel() * 2 // K)
    if N % 16:
        raise ValueError(f"wq describes N = {N} outputs, not a multiple of 16")
    _buf(wq, "wq", N * K // 2, _U8, 16)
    _buf(sw, "sw", 8 * N * ((K // GROUP + 3) // 4), _SW, 8)
    _buf(xq, "xq", M * K // 2, _U8, 16)
    return M, N


def _out_checks(y, M, N, out_dtype, device):
    if y is None:
        return torch.empty((M, N), dtype=out_dtype, device=device)
    _buf(y, "y", M * N * (4 if y.dtype == torch.float32 else 2), (torch.float32, torch.bfloat16))
    return y


def _dump_checks(acc_dump, M, N, K):
    if acc_dump is not None:
        _buf(acc_dump, "acc_dump", 4 * M * N * (K // GROUP), _I32)


def block_map(row_ptr, col_idx, N: int, K: int, bn: int = 64, bk: int = BK, out=None, stream=None):
    """Dense block map int32 [N/bn][K/bk] of a CSR selection: the CSR position of
    each chosen block, -1 elsewhere."""
    nnz = _csr_checks(row_ptr, col_idx, N, bn)
    if K <= 0 or K % bk or N <= 0 or N % bn:
        raise ValueError(f"blocks {bn}x{bk} do not tile a {N}x{K} layer")
    rmap = torch.empty((N // bn, K // bk), dtype=torch.int32, device=row_ptr.device) if out is None \
        else _buf(out, "rmap", 4 * (N // bn) * (K // bk), _I32)
    _on_device(row_ptr=row_ptr, col_idx=col_idx if nnz else None, rmap=rmap)
    _call("mq_block_map", _ptr(row_ptr), _ptr(col_idx) if nnz else None, nnz, N, K, bn, bk, _ptr(rmap),
          _stream(stream))
    return rmap


def gemm_w4a4_residual(xq, sx, wq, sw, row_ptr, col_idx, rq, K: int, bn: int = 64,
                       out_dtype=torch.bfloat16, y=None, acc_dump=None, stream=None, rmap=None):
    """Fused dense + sparse-residual W4A4 GEMM. acc_dump: optional int32 [M][N][K/128].
    rmap: optional block_map(row_ptr, col_idx, ...) of the same selection; the call
    then finds the blocks through it (mq_gemm_w4a4_residual_mapped, same bits)."""
    M, N = _gemm_operands(xq, sx, wq, sw, K)
    nnz = _csr_checks(row_ptr, col_idx, N, bn)
    if nnz:
        _buf(rq, "rq", nnz * bn * BK // 2, _U8, 16)
    y = _out_checks(y, M, N, out_dtype, wq.device)
    _dump_checks(acc_dump, M, N, K)
    if rmap is not None:
        _buf(rmap, "rmap", 4 * (N // bn) * (K // BK), _I32)
        _on_device(xq=xq, sx=sx, wq=wq, sw=sw, rmap=rmap, rq=rq if nnz else None, y=y, acc_dump=acc_dump)
        _call("mq_gemm_w4a4_residual_mapped", _ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), _ptr(rmap),
              _ptr(rq) if nnz else None, nnz, M, N, K, GROUP, bn, BK, _ptr(y), _y_dtype(y.dtype),
              _ptr(acc_dump), _stream(stream))
        return y
    _on_device(xq=xq, sx=sx, wq=wq, sw=sw, row_ptr=row_ptr, col_idx=col_idx if nnz else None,
               rq=rq if nnz else None, y=y, acc_dump=acc_dump)
    _call("mq_gemm_w4a4_residual", _ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), _ptr(row_ptr),
          _ptr(col_idx) if nnz else None, _ptr(rq) if nnz else None, nnz, M, N, K, GROUP, bn, BK,
          _ptr(y), _y_dtype(y.dtype), _ptr(acc_dump), _stream(stream))
    return y


SYNC_WORDS = 544   # MQ_SYNC_WORDS


def sync_words(device="cuda"):
    """The zero-filled int32 [SYNC_WORDS] counter array gemm_w4a4_residual_act needs (one per
    stream of calls; every completed call leaves it zero again)."""
    return torch.zeros(SYNC_WORDS, dtype=torch.int32, device=device)


_ACT_LAUNCH = {"auto": 0, "one": 1, "two": 2}   # MQ_ACT_AUTO, MQ_ACT_ONE_LAUNCH, MQ_ACT_TWO_LAUNCHES


def act_one_launch(M: int, N: int, K: int, launch: str = "auto") -> bool:
    """Whether gemm_w4a4_residual_act runs as one launch ("auto": the library's own
    rule, mq_act_one_launch)."""
    return launch == "one" or (launch == "auto" and _lib.mq_act_one_launch(M, N, K) == 1)


def gemm_w4a4_residual_act(x, wq, sw, rmap, rq, K: int, bn: int = 64, out_dtype=torch.bfloat16, y=None,
                           xq=None, sx=None, sync=None, launch: str = "auto", stream=None):
    """The fused GEMM that quantizes its own activations: x fp32/bf16 [M][K] in,
    y out, plus the codes and scales it used (xq, sx, as quantize_act writes them).
    Returns (y, xq, sx). launch: "one" (M <= 32), "two" (quantize_act, then the
    GEMM) or "auto"; sync: sync_words(), required when one launch runs."""
    if launch not in _ACT_LAUNCH:
        raise ValueError(f"launch must be one of {sorted(_ACT_LAUNCH)}, got {launch!r}")
    M, K2 = _shape2(x, "x")
    if K2 != K:
        raise ValueError(f"x has {K2} inputs, expected K = {K}")
    _x_dtype(x)
    _device_contig(x, "x")
    if xq is None:
        xq = torch.empty((K // GROUP, M, 64), dtype=torch.uint8, device=x.device)
    if sx is None:
        sx = torch.empty(M, dtype=torch.float32, device=x.device)
    _buf(sx, "sx", 4 * M, _F32)
    M2, N = _gemm_operands(xq, sx, wq, sw, K)
    nnz = int(rq.shape[0]) if rq is not None and rq.dim() == 3 else 0
    _buf(rmap, "rmap", 4 * (N // bn) * (K // BK), _I32)
    if nnz:
        _buf(rq, "rq", nnz * bn * BK // 2, _U8, 16)
    y = _out_checks(y, M, N, out_dtype, wq.device)
    if launch == "one" and M > 32:
        raise ValueError("one launch takes at most 32 tokens")
    one = act_one_launch(M, N, K, launch)
    if one:
        if sync is None:
            raise ValueError("sync (sync_words()) is required for the one-launch form")
        _buf(sync, "sync", 4 * SYNC_WORDS, _I32, 4)
    _on_device(x=x, xq=xq, sx=sx, wq=wq, sw=sw, rmap=rmap, rq=rq if nnz else None, y=y,
               sync=sync if one else None)
    _call("mq_gemm_w4a4_residual_act", _ptr(x), _x_dtype(x), _ptr(wq), _ptr(sw), _ptr(rmap),
          _ptr(rq) if nnz else None, nnz, M, N, K, GROUP, bn, BK, _ptr(xq), _ptr(sx),
          _ptr(sync) if one else None, _ACT_LAUNCH[launch], _ptr(y), _y_dtype(y.dtype), _stream(stream))
    return y, xq, sx


READ_PROBE_WORDS = 8192   # MQ_READ_PROBE_WORDS


def read_probe(buf, nbytes: int = None, out=None, stream=None):
    """Streaming read of the first nbytes of buf (a measurement aid: the read rate a
    kernel reaches at that byte count). Returns the uint32 output words."""
    _device_contig(buf, "buf")
    have = buf.numel() * buf.element_size()
    nbytes = have if nbytes is None else int(nbytes)
    if nbytes < 0 or nbytes > have or nbytes % 16:
        raise ValueError(f"nbytes must be a multiple of 16 within the buffer's {have} bytes, got {nbytes}")
    if out is None:
        out = torch.empty(READ_PROBE_WORDS, dtype=torch.int32, device=buf.device)
    _buf(out, "out", 4 * READ_PROBE_WORDS, _I32)
    _on_device(buf=buf, out=out)
    _call("mq_read_probe", _ptr(buf), nbytes, _ptr(out), _stream(stream))
    return out


def gemm_w4a4_dense(xq, sx, wq, sw, K: int, out_dtype=torch.bfloat16, y=None, acc_dump=None,
                    stream=None):
    """Dense-only W4A4 GEMM (the kernel the residual is fused into)."""
    M, N = _gemm_operands(xq, sx, wq, sw, K)
    y = _out_checks(y, M, N, out_dtype, wq.device)
    _dump_checks(acc_dump, M, N, K)
    _on_device(xq=xq, sx=sx, wq=wq, sw=sw, y=y, acc_dump=acc_dump)
    _call("mq_gemm_w4a4_dense", _ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), M, N, K, GROUP, _ptr(y),
          _y_dtype(y.dtype), _ptr(acc_dump), _stream(stream))
    return y


def gemm_residual_separate(xq, sx, wq, sw, row_ptr, col_idx, rq, K: int, bn: int = 64,
                           out_dtype=torch.bfloat16, y=None, ws=None, stream=None):
    """The separate-kernel alternative: dense kernel to fp32 partials `ws`, then a
    residual kernel that re-reads the activations and merges."""
    M, N = _gemm_operands(xq, sx, wq, sw, K)
    nnz = _csr_checks(row_ptr, col_idx, N, bn)
    if nnz:
        _buf(rq, "rq", nnz * bn * BK // 2, _U8, 16)
    y = _out_checks(y, M, N, out_dtype, wq.device)
    if ws is None:
        ws = torch.empty((M, N), dtype=torch.float32, device=wq.device)
    else:
        _buf(ws, "ws", 4 * M * N, _F32)
    _on_device(xq=xq, sx=sx, wq=wq, sw=sw, row_ptr=row_ptr, col_idx=col_idx if nnz else None,
               rq=rq if nnz else None, y=y, ws=ws)
    _call("mq_gemm_residual_separate", _ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), _ptr(row_ptr),
          _ptr(col_idx) if nnz else None, _ptr(rq) if nnz else None, nnz, M, N, K, GROUP, bn, BK,
          _ptr(y), _y_dtype(y.dtype), _ptr(ws), _stream(stream))
    return y


def forward_layer(x, w, k_blocks: int, bn: int = 64, out_dtype=torch.bfloat16, migrate: bool = False,
                  stream=None):
    """The whole path on device: (optional outlier migration) -> h -> select -> pack
    -> quantize X -> fused GEMM."""
    s = r = None
    if migrate:
        s, r = smooth_factors(x, w, stream=stream)
        w = scale_columns(w, s, stream=stream)
    h = hessian_diag(x, r=r, stream=stream)
    row_ptr, col_idx, delta = select_blocks(w, h, k_blocks, bn=bn, stream=stream)
    wq, sw, rq = pack_weights(w, row_ptr, col_idx, bn=bn, stream=stream)
    xq, sx = quantize_act(x, r=r, stream=stream)
    y = gemm_w4a4_residual(xq, sx, wq, sw, row_ptr, col_idx, rq, w.shape[1], bn=bn,
                           out_dtype=out_dtype, stream=stream)
    return dict(h=h, row_ptr=row_ptr, col_idx=col_idx, delta=delta, wq=wq, sw=sw, rq=rq, xq=xq,
                sx=sx, y=y, s=s, r=r, w_hat=w if migrate else None)
