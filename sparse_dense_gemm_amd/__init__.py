"""Python binding of the Spense C interface (``include/spense.h``).

Argument marshalling only: every step of the layer runs in the HIP library
``libspense.so`` built next to this file.  There is no Python or CPU fallback;
if the library is missing every call raises.

Tensors are passed by device pointer (``tensor.data_ptr()``); torch is used
only to own device memory and to name the current HIP stream.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

DT_F32 = 0
DT_BF16 = 1
DT_FP8 = 2

SPENSE_OK = 0
SPENSE_EINVAL = -1
SPENSE_EUNSUPPORTED = -2
SPENSE_ENOMEM = -3
SPENSE_EHIP = -4
SPENSE_ESCRATCH = -5

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspense.so")

_lib_handle = None


class SpenseError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _lib()
        msg = lib.spense_strerror(status).decode()
        if status == SPENSE_EHIP:
            msg += f" (hipError_t {lib.spense_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{status}]")
        self.status = status


class LayerInfo(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("K_s", ctypes.c_int64), ("K_d", ctypes.c_int64),
        ("wdtype", ctypes.c_int32), ("gather", ctypes.c_int32),
        ("weight_bytes", ctypes.c_int64), ("device_bytes", ctypes.c_int64),
        ("split", ctypes.c_int32), ("N_s", ctypes.c_int64), ("N_d", ctypes.c_int64),
    ]


def _lib():
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m sparse_dense_gemm_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.spense_pack.argtypes = [vp, i32, i64, i64, i64, vp, vp, i64, f64, vp, ctypes.POINTER(vp)]
    lib.spense_pack.restype = ctypes.c_int
    lib.spense_pack_rows.argtypes = [vp, i32, i64, i64, i64, vp, vp, i64, f64, vp, ctypes.POINTER(vp)]
    lib.spense_pack_rows.restype = ctypes.c_int
    lib.spense_export_rows.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.spense_export_rows.restype = ctypes.c_int
    lib.spense_pack_glu.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp, vp, vp, i64, f64, vp, ctypes.POINTER(vp)]
    lib.spense_pack_glu.restype = ctypes.c_int
    lib.spense_glu.argtypes = [vp, vp, i64, i64, vp, i64, vp, i32, i64, vp]
    lib.spense_glu.restype = ctypes.c_int
    lib.spense_score_glu.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp, vp, vp, i64, i64, vp, i64, vp, vp]
    lib.spense_score_glu.restype = ctypes.c_int
    lib.spense_select_dense.argtypes = [vp, i64, i64, vp, vp]
    lib.spense_select_dense.restype = ctypes.c_int
    lib.spense_linear.argtypes = [vp, vp, i32, i64, i64, vp, i32, i64, vp]
    lib.spense_linear.restype = ctypes.c_int
    lib.spense_linear_splits.argtypes = [vp, vp, i32, i64, i64, vp, i32, i64, i32, vp]
    lib.spense_linear_noalloc.argtypes = [vp, vp, i32, i64, i64, vp, i32, i64, vp]
    lib.spense_linear_noalloc.restype = ctypes.c_int
    lib.spense_quantize_tokens.restype = ctypes.c_int
    lib.spense_quantize_tokens.argtypes = [vp, i64, i64, i64, vp, i64, vp, vp]
    lib.spense_linear_w8a8.restype = ctypes.c_int
    lib.spense_linear_w8a8.argtypes = [vp, vp, i64, i64, vp, i32, i64, i32, vp]
    lib.spense_linear_splits.restype = ctypes.c_int
    lib.spense_info.argtypes = [vp, ctypes.POINTER(LayerInfo)]
    lib.spense_info.restype = ctypes.c_int
    lib.spense_export.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.spense_export.restype = ctypes.c_int
    lib.spense_free.argtypes = [vp]
    lib.spense_free.restype = ctypes.c_int
    lib.spense_strerror.argtypes = [ctypes.c_int]
    lib.spense_strerror.restype = ctypes.c_char_p
    lib.spense_last_hip_error.argtypes = []
    lib.spense_last_hip_error.restype = ctypes.c_int
    lib.spense_abi_version.argtypes = []
    lib.spense_abi_version.restype = ctypes.c_int
    _lib_handle = lib
    return lib


def _check(status: int, where: str):
    if status != SPENSE_OK:
        raise SpenseError(status, where)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dtype_of(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return DT_F32
    if t.dtype == torch.bfloat16:
        return DT_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return DT_FP8
    raise TypeError(f"unsupported dtype {t.dtype}")


def spense_pack(W, wdtype: Optional[int] = None, *, scales=None, dense_cols=None, dense_fraction: float = 0.0,
                N: Optional[int] = None, K: Optional[int] = None, ldw: Optional[int] = None, stream=None) -> int:
    """Pack a weight matrix; returns the opaque handle (an int)."""
    if wdtype is None:
        wdtype = dtype_of(W)
    if N is None:
        N = W.shape[0]
    if K is None:
        K = W.shape[1]
    if ldw is None:
        ldw = W.stride(0) if hasattr(W, "stride") else K
    cols_ptr = None
    n_dense = 0
    if dense_cols is not None:
        cols = np.ascontiguousarray(np.asarray(dense_cols, dtype=np.int32).ravel())
        n_dense = cols.size
        # an explicit empty set still needs a non-null pointer
        buf = cols if n_dense else np.zeros(1, dtype=np.int32)
        cols_ptr = buf.ctypes.data
    h = ctypes.c_void_p()
    st = _lib().spense_pack(_ptr(W), wdtype, N, K, ldw, _ptr(scales), cols_ptr, n_dense, float(dense_fraction),
                            _stream(stream), ctypes.byref(h))
    _check(st, "spense_pack")
    return h.value


def spense_pack_rows(W, wdtype: Optional[int] = None, *, scales=None, dense_rows=None, dense_fraction: float = 0.0,
                     N: Optional[int] = None, K: Optional[int] = None, ldw: Optional[int] = None,
                     stream=None) -> int:
    """Pack an output-split layer (dense rows | 2:4 rows); returns the opaque handle (an int)."""
    if wdtype is None:
        wdtype = dtype_of(W)
    if N is None:
        N = W.shape[0]
    if K is None:
        K = W.shape[1]
    if ldw is None:
        ldw = W.stride(0) if hasattr(W, "stride") else K
    rows_ptr = None
    n_dense = 0
    if dense_rows is not None:
        rows = np.ascontiguousarray(np.asarray(dense_rows, dtype=np.int32).ravel())
        n_dense = rows.size
        buf = rows if n_dense else np.zeros(1, dtype=np.int32)
        rows_ptr = buf.ctypes.data
    h = ctypes.c_void_p()
    st = _lib().spense_pack_rows(_ptr(W), wdtype, N, K, ldw, _ptr(scales), rows_ptr, n_dense, float(dense_fraction),
                                 _stream(stream), ctypes.byref(h))
    _check(st, "spense_pack_rows")
    return h.value


def spense_export_rows(h: int, vals=None, meta=None, mask=None, dense=None, stream=None) -> np.ndarray:
    """Write an output-split layer's canonical form into the given device tensors; returns rho (numpy int32)."""
    info = spense_info(h)
    rho = np.empty(info["N"], dtype=np.int32)
    st = _lib().spense_export_rows(h, _ptr(vals), _ptr(meta), _ptr(mask), _ptr(dense), rho.ctypes.data,
                                   _stream(stream))
    _check(st, "spense_export_rows")
    return rho


def spense_pack_glu(W_gu, W_down, wdtype: int, *, H: int, I: int, s_gu=None, s_down=None, dense_idx=None,
                    dense_fraction: float = 0.0, stream=None) -> int:
    """Pack a GLU block: W_gu = [gate; up] as [2I, H], W_down [H, I]; returns the handle."""
    idx_ptr, n_dense = None, 0
    if dense_idx is not None:
        idx = np.ascontiguousarray(np.asarray(dense_idx, dtype=np.int32).ravel())
        n_dense = idx.size
        buf = idx if n_dense else np.zeros(1, dtype=np.int32)
        idx_ptr = buf.ctypes.data
    ld_gu = W_gu.stride(0) if hasattr(W_gu, "stride") else H
    ld_down = W_down.stride(0) if hasattr(W_down, "stride") else I
    h = ctypes.c_void_p()
    st = _lib().spense_pack_glu(_ptr(W_gu), _ptr(W_down), wdtype, H, I, ld_gu, ld_down, _ptr(s_gu), _ptr(s_down),
                                idx_ptr, n_dense, float(dense_fraction), _stream(stream), ctypes.byref(h))
    _check(st, "spense_pack_glu")
    return h.value


def spense_glu(h: int, X, A, Y, *, M: Optional[int] = None, stream=None) -> None:
    """GLU block forward: A (bf16 [M, >= I]) receives silu(gate) * up in rho order, Y the block output."""
    M = X.shape[0] if M is None else M
    ydtype = dtype_of(Y)
    st = _lib().spense_glu(h, _ptr(X), M, X.stride(0), _ptr(A), A.stride(0), _ptr(Y), ydtype, Y.stride(0),
                           _stream(stream))
    _check(st, "spense_glu")


def spense_score_glu(W_gu, W_down, wdtype: int, *, H: int, I: int, X_cal, A_cal, score, s_gu=None, s_down=None,
                     stream=None) -> None:
    """SpenseGPT+ scores of the intermediate indices of a GLU block into `score` (float32 [I], device)."""
    ld_gu = W_gu.stride(0) if hasattr(W_gu, "stride") else H
    ld_down = W_down.stride(0) if hasattr(W_down, "stride") else I
    st = _lib().spense_score_glu(_ptr(W_gu), _ptr(W_down), wdtype, H, I, ld_gu, ld_down, _ptr(s_gu), _ptr(s_down),
                                 _ptr(X_cal), X_cal.shape[0], X_cal.stride(0), _ptr(A_cal), A_cal.stride(0),
                                 _ptr(score), _stream(stream))
    _check(st, "spense_score_glu")


def spense_select_dense(score, k: int, stream=None) -> np.ndarray:
    """Indices of the k highest scores (ties to the lower index), ascending, as numpy int32."""
    out = np.zeros(max(k, 1), dtype=np.int32)
    st = _lib().spense_select_dense(_ptr(score), score.numel(), k, out.ctypes.data, _stream(stream))
    _check(st, "spense_select_dense")
    return out[:k]


def spense_linear(h: int, X, Y, *, xdtype: Optional[int] = None, ydtype: Optional[int] = None,
                  M: Optional[int] = None, ldx: Optional[int] = None, ldy: Optional[int] = None, stream=None) -> None:
    """Y = X . W^T through the packed layer (asynchronous on the stream)."""
    spense_linear_splits(h, X, Y, 0, xdtype=xdtype, ydtype=ydtype, M=M, ldx=ldx, ldy=ldy, stream=stream)


def spense_linear_splits(h: int, X, Y, splits: int, *, xdtype: Optional[int] = None, ydtype: Optional[int] = None,
                         M: Optional[int] = None, ldx: Optional[int] = None, ldy: Optional[int] = None,
                         stream=None) -> None:
    if xdtype is None:
        xdtype = dtype_of(X)
    if ydtype is None:
        ydtype = dtype_of(Y)
    if M is None:
        M = X.shape[0]
    if ldx is None:
        ldx = X.stride(0)
    if ldy is None:
        ldy = Y.stride(0)
    st = _lib().spense_linear_splits(h, _ptr(X), xdtype, M, ldx, _ptr(Y), ydtype, ldy, splits, _stream(stream))
    _check(st, "spense_linear")


def spense_linear_noalloc(h: int, X, Y, *, xdtype: Optional[int] = None, ydtype: Optional[int] = None,
                          M: Optional[int] = None, ldx: Optional[int] = None, ldy: Optional[int] = None,
                          stream=None) -> None:
    """spense_linear with its workspaces in the library's fixed device scratch (allocates nothing)."""
    xdtype = dtype_of(X) if xdtype is None else xdtype
    ydtype = dtype_of(Y) if ydtype is None else ydtype
    M = X.shape[0] if M is None else M
    ldx = X.stride(0) if ldx is None else ldx
    ldy = Y.stride(0) if ldy is None else ldy
    st = _lib().spense_linear_noalloc(h, _ptr(X), xdtype, M, ldx, _ptr(Y), ydtype, ldy, _stream(stream))
    _check(st, "spense_linear_noalloc")


def spense_quantize_tokens(X, Xq, sx, *, M: Optional[int] = None, K: Optional[int] = None,
                           ldx: Optional[int] = None, ldq: Optional[int] = None, stream=None) -> None:
    """Per-token e4m3 codes of bf16 X into Xq (uint8 [M, K]) and the token scales into sx (float32 [M])."""
    if M is None:
        M = X.shape[0]
    if K is None:
        K = X.shape[1]
    if ldx is None:
        ldx = X.stride(0)
    if ldq is None:
        ldq = Xq.stride(0)
    st = _lib().spense_quantize_tokens(_ptr(X), M, K, ldx, _ptr(Xq), ldq, _ptr(sx), _stream(stream))
    _check(st, "spense_quantize_tokens")


def spense_linear_w8a8(h: int, X, Y, *, splits: int = 0, ydtype: Optional[int] = None, M: Optional[int] = None,
                       ldx: Optional[int] = None, ldy: Optional[int] = None, stream=None) -> None:
    """Y = (per-token e4m3 X) . W^T on an e4m3 input-split layer (asynchronous on the stream)."""
    if ydtype is None:
        ydtype = dtype_of(Y)
    if M is None:
        M = X.shape[0]
    if ldx is None:
        ldx = X.stride(0)
    if ldy is None:
        ldy = Y.stride(0)
    st = _lib().spense_linear_w8a8(h, _ptr(X), M, ldx, _ptr(Y), ydtype, ldy, splits, _stream(stream))
    _check(st, "spense_linear_w8a8")


def spense_info(h: int) -> dict:
    info = LayerInfo()
    _check(_lib().spense_info(h, ctypes.byref(info)), "spense_info")
    return {f: getattr(info, f) for f, _ in LayerInfo._fields_}


def spense_export(h: int, vals=None, meta=None, mask=None, dense=None, stream=None) -> np.ndarray:
    """Write the canonical packed form into the given device tensors; returns pi (numpy int32)."""
    info = spense_info(h)
    pi = np.empty(info["K"], dtype=np.int32)
    st = _lib().spense_export(h, _ptr(vals), _ptr(meta), _ptr(mask), _ptr(dense), pi.ctypes.data, _stream(stream))
    _check(st, "spense_export")
    return pi


def spense_free(h: int) -> None:
    _check(_lib().spense_free(h), "spense_free")


def spense_abi_version() -> int:
    return _lib().spense_abi_version()


class SpenseLinear:
    """Owns one packed layer; ``layer(X, Y)`` runs spense_linear."""

    def __init__(self, W, wdtype: Optional[int] = None, **kw):
        self.handle = spense_pack(W, wdtype, **kw)
        self.info = spense_info(self.handle)

    def __call__(self, X, Y, splits: int = 0, stream=None):
        spense_linear_splits(self.handle, X, Y, splits, stream=stream)
        return Y

    def close(self):
        if self.handle:
            spense_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
