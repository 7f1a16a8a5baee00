"""weight_only_quant_amd — Python binding of the qmat C ABI (include/qmat.h).

Argument marshalling only: every step of the product runs in the HIP library
(libqmat.so, built for gfx950).  Host arrays are numpy; device buffers are torch
tensors (PyTorch supplies device memory and streams, nothing else).  The names are
those of the C functions.  If the library is missing, importing a function raises:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmat.so")

QMAT_OK, QMAT_EINVAL, QMAT_ESHAPE, QMAT_ERANGE, QMAT_ESIZE, QMAT_EHIP, QMAT_ENOMEM = range(7)
QMAT_Q4, QMAT_Q5, QMAT_Q6, QMAT_FP8_E4M3_ROW, QMAT_Q8 = 4, 5, 6, 8, 9
QMAT_ROUTE_AUTO, QMAT_ROUTE_VALU, QMAT_ROUTE_MFMA, QMAT_ROUTE_GEMM, QMAT_ROUTE_MFMA_OFFSET = 0, 1, 2, 3, 4
QMAT_ENCODE_RTN, QMAT_ENCODE_GROUPED_SEARCH = 0, 1
FORMATS = (QMAT_Q4, QMAT_Q5, QMAT_Q6, QMAT_FP8_E4M3_ROW, QMAT_Q8)
MAX_T = 16

# C function name -> (restype, argtypes)
_i64, _vp, _int, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "qmat_packed_bytes": (_sz, [_int, _i64, _i64]),
    "qmat_pack": (_int, [_int, _i64, _i64, _vp, _vp, _vp, _sz]),
    "qmat_quantize": (_int, [_int, _i64, _i64, _vp, _vp, _int, _vp, _vp]),
    "qmat_create": (_int, [ctypes.POINTER(_vp), _int, _i64, _i64, _vp, _sz]),
    "qmat_create_view": (_int, [ctypes.POINTER(_vp), _vp, _i64, _i64]),
    "qmat_run": (_int, [_vp, _vp, _vp, _int, _vp]),
    "qmat_run_static": (_int, [_int, _i64, _i64, _vp, _sz, _vp, _vp, _int, _vp]),
    "qmat_run_ex": (_int, [_vp, _vp, _vp, _int, _int, _int, _int, _int, _vp]),
    "qmat_dequant": (_int, [_vp, _vp, _vp]),
    "qmat_run_plan": (_int, [_vp, _vp, _vp, _int, _vp, _vp]),
    "qmat_get_plan": (_int, [_vp, _int, _int, _vp]),
    "qmat_workspace_bytes": (_sz, [_vp, _int]),
    "qmat_destroy": (None, [_vp]),
    "qmat_last_error": (ctypes.c_char_p, []),
    "qmat_logits_create": (_int, [ctypes.POINTER(_vp), _i64, _int, _int]),
    "qmat_logits_run": (_int, [_vp, _vp, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp]),
    "qmat_logits_destroy": (None, [_vp]),
    "qmat_run_logits": (_int, [_vp, _vp, _vp, _vp, _int, _int, _vp, _vp, _vp, _vp, _vp]),
}


class QmatError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"qmat status {status}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded libqmat.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(hipcc --offload-arch=gfx950); there is no non-HIP path")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != QMAT_OK:
        raise QmatError(status, qmat_last_error())


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def qmat_last_error() -> str:
    return lib().qmat_last_error().decode()


def qmat_packed_bytes(fmt: int, M: int, K: int) -> int:
    return int(lib().qmat_packed_bytes(fmt, M, K))


def qmat_pack(fmt: int, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Host pack.  Groupwise: codes int8 [M,K], scales uint16 binary16 bits [M,K/64];
    FP8: codes uint8 E4M3 bytes [M,K], scales float32 [M].  Returns uint8 [packed_bytes]."""
    if fmt == QMAT_FP8_E4M3_ROW:
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.float32)
    else:
        codes = np.ascontiguousarray(codes, dtype=np.int8)
        scales = np.ascontiguousarray(scales, dtype=np.uint16)
    if codes.ndim != 2:
        raise ValueError("codes must be 2-D [M, K]")
    M, K = codes.shape
    want = (M,) if fmt == QMAT_FP8_E4M3_ROW else (M, K // 64)
    if scales.shape != want:
        raise ValueError(f"scales must have shape {want}")
    n = qmat_packed_bytes(fmt, M, K)
    out = np.empty(max(n, 1), dtype=np.uint8)
    _check(lib().qmat_pack(fmt, M, K, codes.ctypes.data, scales.ctypes.data, out.ctypes.data, n))
    return out[:n]


def qmat_quantize(fmt: int, w: np.ndarray, importance: Optional[np.ndarray] = None,
                  encoder: int = QMAT_ENCODE_RTN):
    """Host encoder: float32 w [M, K] -> (codes, scales) as qmat_pack takes them
    (groupwise: int8 [M, K], uint16 [M, K/64]; FP8: uint8 [M, K], float32 [M])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D [M, K]")
    M, K = w.shape
    imp = None if importance is None else np.ascontiguousarray(importance, dtype=np.float32)
    if imp is not None and imp.shape != (K,):
        raise ValueError("importance must be [K]")
    if fmt == QMAT_FP8_E4M3_ROW:
        codes, scales = np.empty((M, K), np.uint8), np.empty((M,), np.float32)
    else:
        codes, scales = np.empty((M, K), np.int8), np.empty((M, max(K // 64, 1)), np.uint16)
    _check(lib().qmat_quantize(fmt, M, K, w.ctypes.data, None if imp is None else imp.ctypes.data, encoder,
                               codes.ctypes.data, scales.ctypes.data))
    return codes, scales


def qmat_create(fmt: int, M: int, K: int, packed_dev) -> int:
    """packed_dev: a torch uint8 device tensor holding qmat_pack's output (borrowed)."""
    h = ctypes.c_void_p()
    _check(lib().qmat_create(ctypes.byref(h), fmt, M, K, packed_dev.data_ptr(), packed_dev.numel()))
    return h.value


def qmat_create_view(parent: int, row0: int, rows: int) -> int:
    """A handle over rows [row0, row0 + rows) of parent's matrix (row0 a multiple of 64)."""
    h = ctypes.c_void_p()
    _check(lib().qmat_create_view(ctypes.byref(h), parent, row0, rows))
    return h.value


def qmat_run(handle: int, x, y, T: Optional[int] = None, stream=None) -> None:
    """x: bf16 device [T,K]; y: fp32 device [T,M]."""
    T = x.shape[0] if T is None else T
    _check(lib().qmat_run(handle, x.data_ptr(), y.data_ptr(), T, _stream_handle(stream)))


def qmat_run_static(fmt: int, M: int, K: int, packed_dev, x, y, T: Optional[int] = None, stream=None) -> None:
    """qmat_run without a handle or any allocation: packed_dev is a torch uint8 device tensor
    holding qmat_pack's output; x bf16 device [T,K]; y fp32 device [T,M]."""
    T = x.shape[0] if T is None else T
    _check(lib().qmat_run_static(fmt, M, K, packed_dev.data_ptr(), packed_dev.numel(), x.data_ptr(), y.data_ptr(), T,
                                 _stream_handle(stream)))


def qmat_run_ex(handle: int, x, y, T: Optional[int] = None, route: int = QMAT_ROUTE_AUTO,
                waves: int = 0, splits: int = 0, stream=None, depth: int = 0) -> None:
    T = x.shape[0] if T is None else T
    _check(lib().qmat_run_ex(handle, x.data_ptr(), y.data_ptr(), T, route, depth, waves, splits,
                             _stream_handle(stream)))


def qmat_dequant(handle: int, w, stream=None) -> None:
    """w: fp32 device [M,K]."""
    _check(lib().qmat_dequant(handle, w.data_ptr(), _stream_handle(stream)))


class qmat_plan(ctypes.Structure):
    """The C struct qmat_plan (launch shape of the product kernel)."""
    _fields_ = [("route", _int), ("depth", _int), ("waves", _int), ("splits", _int),
                ("tail_tiles", _int), ("tail_splits", _int), ("tiles", _int)]

    def as_tuple(self):
        return (self.route, self.depth, self.waves, self.splits, self.tail_tiles, self.tail_splits, self.tiles)


def qmat_get_plan(handle: int, T: int, route: int = QMAT_ROUTE_AUTO) -> qmat_plan:
    """The qmat_plan qmat_run would use for T tokens on a route."""
    p = qmat_plan()
    _check(lib().qmat_get_plan(handle, T, route, ctypes.byref(p)))
    return p


def qmat_run_plan(handle: int, x, y, plan: qmat_plan, T: Optional[int] = None, stream=None) -> None:
    """qmat_run with an explicit qmat_plan."""
    T = x.shape[0] if T is None else T
    _check(lib().qmat_run_plan(handle, x.data_ptr(), y.data_ptr(), T, ctypes.byref(plan), _stream_handle(stream)))


def qmat_workspace_bytes(handle: int, T: int = 0) -> int:
    """Device workspace bytes the automatic plan uses at T tokens (T = 0: all the handle holds)."""
    return int(lib().qmat_workspace_bytes(handle, T))


def qmat_destroy(handle: Optional[int]) -> None:
    if handle:
        lib().qmat_destroy(handle)


def qmat_logits_create(M: int, max_T: int, max_k: int) -> int:
    """Epilogue handle for M logit rows, up to max_T tokens and top-k up to max_k."""
    h = ctypes.c_void_p()
    _check(lib().qmat_logits_create(ctypes.byref(h), M, max_T, max_k))
    return h.value


def qmat_logits_run(handle: int, y, k: int, lse=None, top_vals=None, top_ids=None, index=None,
                    T: Optional[int] = None, stream=None) -> None:
    """y: fp32 device [T, >= M] (row stride y.stride(0)); lse fp32 [T]; top_vals fp32 [T, k];
    top_ids int32 [T, k]; index int32 [M] or None."""
    T = y.shape[0] if T is None else T
    ptr = lambda a: None if a is None else a.data_ptr()
    _check(lib().qmat_logits_run(handle, y.data_ptr(), y.stride(0), T, k, ptr(index), ptr(lse), ptr(top_vals),
                                 ptr(top_ids), _stream_handle(stream)))


def qmat_run_logits(handle: int, epilogue: int, x, k: int, y=None, lse=None, top_vals=None, top_ids=None,
                    index=None, T: Optional[int] = None, stream=None) -> None:
    """Product, then epilogue, in one call: x bf16
    device [T, K]; y fp32 device [T, M] or None; lse fp32 [T]; top_vals fp32 [T, k]; top_ids int32
    [T, k]; index int32 [M] or None."""
    T = x.shape[0] if T is None else T
    ptr = lambda a: None if a is None else a.data_ptr()
    _check(lib().qmat_run_logits(handle, epilogue, x.data_ptr(), ptr(y), T, k, ptr(index), ptr(lse), ptr(top_vals),
                                 ptr(top_ids), _stream_handle(stream)))


def qmat_logits_destroy(handle: Optional[int]) -> None:
    if handle:
        lib().qmat_logits_destroy(handle)


class QMat:
    """A packed matrix resident on the GPU plus its library handle.

    Holds the device copy of the packed blob (the handle borrows it)."""

    def __init__(self, fmt: int, codes: np.ndarray, scales: np.ndarray, device: str = "cuda"):
        import torch
        self.fmt = fmt
        self.M, self.K = codes.shape
        packed = qmat_pack(fmt, codes, scales)
        self.packed = torch.from_numpy(packed).to(device)
        self.handle = qmat_create(fmt, self.M, self.K, self.packed)

    @classmethod
    def from_packed(cls, fmt: int, M: int, K: int, packed_dev):
        self = cls.__new__(cls)
        self.fmt, self.M, self.K = fmt, M, K
        self.packed = packed_dev
        self.handle = qmat_create(fmt, M, K, packed_dev)
        return self

    def run(self, x, y=None, route: int = QMAT_ROUTE_AUTO, waves: int = 0, splits: int = 0, stream=None,
            depth: int = 0):
        import torch
        if y is None:
            y = torch.empty((x.shape[0], self.M), dtype=torch.float32, device=x.device)
        if route == QMAT_ROUTE_AUTO and not (waves or splits or depth):
            qmat_run(self.handle, x, y, stream=stream)
        else:
            qmat_run_ex(self.handle, x, y, route=route, waves=waves, splits=splits, stream=stream, depth=depth)
        return y

    def dequant(self, w=None, stream=None):
        import torch
        if w is None:
            w = torch.empty((self.M, self.K), dtype=torch.float32, device=self.packed.device)
        qmat_dequant(self.handle, w, stream=stream)
        return w

    def close(self):
        qmat_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                self.close()
        except Exception:
            pass
