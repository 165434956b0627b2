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
    "mq_select_blocks": [_p, _p, _i64, _i64, _int, _int, _int, _i64, _p, _p, _p, _p, C.c_size_t, _p],
    "mq_pack_weights": [_p, _i64, _i64, _int, _int, _int, _p, _p, _i64, _p, _p, _p, _p],
    "mq_gemm_w4a4_residual": [_p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _int, _int, _int,
                              _p, _int, _p, _p, C.c_size_t, _p],
    "mq_gemm_w4a4_dense": [_p, _p, _p, _p, _i64, _i64, _i64, _int, _p, _int, _p, _p, C.c_size_t, _p],
    "mq_gemm_residual_separate": [_p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _int, _int,
                                  _int, _p, _int, _p, _p, C.c_size_t, _p],
}
for _name, _args in _SIGS.items():
    getattr(_lib, _name).argtypes = _args
    getattr(_lib, _name).restype = C.c_int
_lib.mq_status_string.argtypes = [C.c_int]
_lib.mq_status_string.restype = C.c_char_p
_lib.mq_version.argtypes = []
_lib.mq_version.restype = C.c_int
_lib.mq_gemm_workspace_bytes.argtypes = [_i64, _i64, _i64]
_lib.mq_gemm_workspace_bytes.restype = C.c_size_t
_lib.mq_select_workspace_bytes.argtypes = [_i64, _i64, _int, _int]
_lib.mq_select_workspace_bytes.restype = C.c_size_t

EXPORTS = tuple(_SIGS) + ("mq_status_string", "mq_version", "mq_gemm_workspace_bytes",
                          "mq_select_workspace_bytes")


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
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# --------------------------------------------------------------------------- a0
def hessian_diag(x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    _device_contig(x, "x")
    M, K = x.shape
    h = torch.empty(K, dtype=torch.float32, device=x.device) if out is None else out
    _call("mq_hessian_diag", _ptr(x), _x_dtype(x), M, K, _ptr(h), _stream(stream))
    return h


# --------------------------------------------------------------------------- a4
def quantize_act(x: torch.Tensor, xq: torch.Tensor | None = None, sx: torch.Tensor | None = None,
                 stream=None):
    """Returns (xq u8 [K/128][M][64], sx fp32 [M])."""
    _device_contig(x, "x")
    M, K = x.shape
    if xq is None:
        xq = torch.empty((K // GROUP, M, 64), dtype=torch.uint8, device=x.device)
    if sx is None:
        sx = torch.empty(M, dtype=torch.float32, device=x.device)
    _call("mq_quantize_act", _ptr(x), _x_dtype(x), M, K, _ptr(xq), _ptr(sx), _stream(stream))
    return xq, sx


# --------------------------------------------------------------------------- a2
def select_workspace(N: int, K: int, bn: int = 64, bk: int = BK, device="cuda"):
    """Scratch for select_blocks (per-block ranks), so the call allocates nothing."""
    n = int(_lib.mq_select_workspace_bytes(N, K, bn, bk))
    return torch.empty(max(n, 4), dtype=torch.uint8, device=device)


def select_blocks(w: torch.Tensor, h: torch.Tensor, k_blocks: int, bn: int = 64, group: int = GROUP,
                  bk: int = BK, out=None, workspace=None, stream=None):
    """Returns (row_ptr int32 [N/bn+1], col_idx int32 [k_blocks], delta fp64 [NB]).
    workspace: optional select_workspace(...) tensor; without it the library takes a
    stream-ordered allocation for the call."""
    _device_contig(w, "w")
    _device_contig(h, "h")
    N, K = w.shape
    nb = (N // bn) * (K // bk)
    if out is None:
        row_ptr = torch.empty(N // bn + 1, dtype=torch.int32, device=w.device)
        col_idx = torch.empty(max(k_blocks, 1), dtype=torch.int32, device=w.device)
        delta = torch.empty(max(nb, 1), dtype=torch.float64, device=w.device)
    else:
        row_ptr, col_idx, delta = out
    ws = _ptr(workspace) if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _call("mq_select_blocks", _ptr(w), _ptr(h), N, K, group, bn, bk, k_blocks, _ptr(row_ptr),
          _ptr(col_idx), _ptr(delta), ws, wsb, _stream(stream))
    return row_ptr, col_idx[:k_blocks], delta[:nb]


# --------------------------------------------------------------------------- a1 + a3
def pack_weights(w: torch.Tensor, row_ptr: torch.Tensor, col_idx: torch.Tensor, bn: int = 64,
                 group: int = GROUP, bk: int = BK, out=None, stream=None):
    """Returns (wq u8 [N/16][G][1024], sw fp16-bits int16 [N/16][G4][16][4],
    rq u8 [nnz][bn][bk/2]) with G = K/128, G4 = ceil(G/4)."""
    _device_contig(w, "w")
    N, K = w.shape
    nnz = int(col_idx.numel())
    if out is None:
        G = K // group
        wq = torch.empty((N // 16, G, 1024), dtype=torch.uint8, device=w.device)
        sw = torch.empty((N // 16, (G + 3) // 4, 16, 4), dtype=torch.int16, device=w.device)
        rq = torch.empty((max(nnz, 1), bn, bk // 2), dtype=torch.uint8, device=w.device)
    else:
        wq, sw, rq = out
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


def _gemm_mn(sx, wq, K: int):
    """(M, N) of a GEMM call: M tokens from sx, N outputs from the packed weight bytes."""
    if K <= 0 or (wq.numel() * 2) % K:
        raise ValueError(f"wq holds {wq.numel()} bytes, not a multiple of K/2 = {K // 2}")
    return int(sx.numel()), int(wq.numel() * 2 // K)


def workspace_bytes(M: int, N: int, K: int) -> int:
    """Device bytes of split-K partials the GEMM calls need for this shape."""
    return int(_lib.mq_gemm_workspace_bytes(M, N, K))


def workspace(M: int, N: int, K: int, device="cuda"):
    """A workspace tensor for the GEMM calls of this shape (None if none is needed)."""
    n = workspace_bytes(M, N, K)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def _ws_args(workspace_t, M, N, K, device):
    if workspace_t is None:
        workspace_t = workspace(M, N, K, device)
    if workspace_t is None:
        return None, 0, None
    return _ptr(workspace_t), workspace_t.numel() * workspace_t.element_size(), workspace_t


def gemm_w4a4_residual(xq, sx, wq, sw, row_ptr, col_idx, rq, K: int, bn: int = 64,
                       out_dtype=torch.bfloat16, y=None, acc_dump=None, workspace=None,
                       stream=None):
    """Fused dense + sparse-residual W4A4 GEMM. acc_dump: optional int32 [M][N][K/128]."""
    M, N = _gemm_mn(sx, wq, K)
    nnz = int(col_idx.numel())
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=wq.device)
    wp, wb, _keep = _ws_args(workspace, M, N, K, wq.device)
    _call("mq_gemm_w4a4_residual", _ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), _ptr(row_ptr),
          _ptr(col_idx) if nnz else None, _ptr(rq) if nnz else None, nnz, M, N, K, GROUP, bn, BK,
          _ptr(y), _y_dtype(y.dtype), _ptr(acc_dump), wp, wb, _stream(stream))
    return y


def gemm_w4a4_dense(xq, sx, wq, sw, K: int, out_dtype=torch.bfloat16, y=None, acc_dump=None,
                    workspace=None, stream=None):
    M, N = _gemm_mn(sx, wq, K)
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=wq.device)
    wp, wb, _keep = _ws_args(workspace, M, N, K, wq.device)
    _call("mq_gemm_w4a4_dense", _ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), M, N, K, GROUP, _ptr(y),
          _y_dtype(y.dtype), _ptr(acc_dump), wp, wb, _stream(stream))
    return y


def gemm_residual_separate(xq, sx, wq, sw, row_ptr, col_idx, rq, K: int, bn: int = 64,
                           out_dtype=torch.bfloat16, y=None, ws=None, workspace=None, stream=None):
    M, N = _gemm_mn(sx, wq, K)
    nnz = int(col_idx.numel())
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=wq.device)
    if ws is None:
        ws = torch.empty((M, N), dtype=torch.float32, device=wq.device)
    wp, wb, _keep = _ws_args(workspace, M, N, K, wq.device)
    _call("mq_gemm_residual_separate", _ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), _ptr(row_ptr),
          _ptr(col_idx) if nnz else None, _ptr(rq) if nnz else None, nnz, M, N, K, GROUP, bn, BK,
          _ptr(y), _y_dtype(y.dtype), _ptr(ws), wp, wb, _stream(stream))
    return y


def forward_layer(x, w, k_blocks: int, bn: int = 64, out_dtype=torch.bfloat16, stream=None):
    """The whole path on device: h -> select -> pack -> quantize X -> fused GEMM."""
    h = hessian_diag(x, stream=stream)
    row_ptr, col_idx, delta = select_blocks(w, h, k_blocks, bn=bn, stream=stream)
    wq, sw, rq = pack_weights(w, row_ptr, col_idx, bn=bn, stream=stream)
    xq, sx = quantize_act(x, stream=stream)
    y = gemm_w4a4_residual(xq, sx, wq, sw, row_ptr, col_idx, rq, w.shape[1], bn=bn,
                           out_dtype=out_dtype, stream=stream)
    return dict(h=h, row_ptr=row_ptr, col_idx=col_idx, delta=delta, wq=wq, sw=sw, rq=rq, xq=xq,
                sx=sx, y=y)
