"""CPU oracle for the weight-only quantized product — TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and the CPU-baseline leg of bench.py may
import this package.  The product library never calls it: it is the independent
reference the GPU results are compared against.  It shares no code with the GPU
path; the only shared module is ``qmat_inputs`` (seeded random draws).

The arithmetic lives in ``qmat_oracle.c`` (plain C, double precision, threaded over
rows); this module only loads it and marshals numpy arrays.

Functions and the definitions they follow (NInfer model cards):
  half_to_double / bf16_to_double / e4m3_to_double   IEEE binary16, bfloat16, OCP E4M3FN
  double_to_half                                      binary16 round-to-nearest-even
  dequant_groupwise   "Qwen3.8-27B for NInfer on the RTX 3090" / "What is different
                      from the upstream artifact": weight = FP16 group scale x code,
                      64-weight groups, negative scales allowed (4, 5, 6 or 8 bits;
                      8-bit groupwise is the cards' Q8 head / projection format)
  dequant_fp8         "Qwen3.8-27B NVFP4 for NInfer" / "Artifact": row-scaled FP8
  gemv                y = x W^T in double, plus A = sum |w x|
  rtn_encode          the upstream round-to-nearest encoder (scale = absmax / qmax)
  grouped_search_encode  the card's encoder: FP16 scale searched over 50 candidates (both
                      signs) for the least importance-weighted squared error
  float_to_e4m3 / fp8_row_encode  E4M3 nearest-even (saturating) and the row-scaled FP8
                      encoding (r = absmax / 448)
  check               the acceptance test |y - y_ref| <= 1e-4 * A + 1e-6
  logsumexp           log sum_i exp(y_i) per token over the output-head logits (the fork's
                      "single-pass logsumexp": giveen/ninfer-ext README, upstream pull
                      requests merged ahead of upstream), in float64 (numpy)
  topk                the k largest logits per token, ties to the lower row, rows mapped
                      through an optional index (the candidate top-k that reads the full head or
                      the indexed 131,072-row proposal head: "Qwen3.8-27B for NInfer on the RTX
                      3090", run notes), numpy
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmat_oracle.c")
_LIB = os.path.join(_HERE, "libqmat_oracle.so")

REL_TOL = 1e-4
ABS_TOL = 1e-6


def build() -> str:
    """Compile the oracle with gcc (-O2, no fast-math: IEEE semantics are required)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
           "-o", _LIB + ".tmp", _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.qo_half_to_double.restype = ctypes.c_double
        L.qo_half_to_double.argtypes = [ctypes.c_uint16]
        L.qo_bf16_to_double.restype = ctypes.c_double
        L.qo_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.qo_e4m3_to_double.restype = ctypes.c_double
        L.qo_e4m3_to_double.argtypes = [ctypes.c_uint8]
        L.qo_double_to_half_rne.restype = ctypes.c_uint16
        L.qo_double_to_half_rne.argtypes = [ctypes.c_double]
        L.qo_dequant_groupwise.restype = i32
        L.qo_dequant_groupwise.argtypes = [i32, i64, i64, vp, vp, vp]
        L.qo_dequant_fp8.restype = i32
        L.qo_dequant_fp8.argtypes = [i64, i64, vp, vp, vp]
        L.qo_gemv.restype = i32
        L.qo_gemv.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, i64, vp, vp, i32]
        L.qo_rtn_encode.restype = i32
        L.qo_rtn_encode.argtypes = [i32, i64, vp, vp, vp]
        L.qo_grouped_search_encode.restype = i32
        L.qo_grouped_search_encode.argtypes = [i32, i64, vp, vp, vp, vp]
        L.qo_float_to_e4m3_rne_sat.restype = ctypes.c_uint8
        L.qo_float_to_e4m3_rne_sat.argtypes = [ctypes.c_float]
        L.qo_fp8_row_encode.restype = i32
        L.qo_fp8_row_encode.argtypes = [i64, i64, vp, vp, vp]
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(st: int, what: str):
    if st != 0:
        raise OracleError(f"{what}: status {st} ({'range' if st == -2 else 'invalid'})")


def half_to_double(h: int) -> float:
    return lib().qo_half_to_double(int(h))


def bf16_to_double(b: int) -> float:
    return lib().qo_bf16_to_double(int(b))


def e4m3_to_double(b: int) -> float:
    return lib().qo_e4m3_to_double(int(b))


def double_to_half(v: float) -> int:
    return int(lib().qo_double_to_half_rne(float(v)))


def dequant_groupwise(bits: int, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    M, K = codes.shape
    if scales.shape != (M, K // 64):
        raise ValueError("scales must be [M, K/64]")
    w = np.empty((M, K), dtype=np.float32)
    _check(lib().qo_dequant_groupwise(bits, M, K, _ptr(codes), _ptr(scales), _ptr(w)), "dequant")
    return w


def dequant_fp8(bytes_: np.ndarray, row_scales: np.ndarray) -> np.ndarray:
    bytes_ = np.ascontiguousarray(bytes_, dtype=np.uint8)
    r = np.ascontiguousarray(row_scales, dtype=np.float32)
    M, K = bytes_.shape
    if r.shape != (M,):
        raise ValueError("row scales must be [M]")
    w = np.empty((M, K), dtype=np.float32)
    _check(lib().qo_dequant_fp8(M, K, _ptr(bytes_), _ptr(r), _ptr(w)), "dequant_fp8")
    return w


def gemv(fmt: int, codes: np.ndarray, scales: np.ndarray, x: np.ndarray,
         rows: Optional[Sequence[int]] = None, nthreads: Optional[int] = None):
    """Returns (y, A), both float64 [T, nrows]: y = x W^T over the requested rows (all
    rows if None), A = sum_j |w_ij x_tj|.  fmt: 4, 5, 6 groupwise with that many bits,
    9 groupwise 8-bit, 8 row-scaled FP8."""
    if fmt == 8:
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.float32)
    else:
        codes = np.ascontiguousarray(codes, dtype=np.int8)
        scales = np.ascontiguousarray(scales, dtype=np.uint16)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    M, K = codes.shape
    T = x.shape[0]
    if x.shape != (T, K):
        raise ValueError("x must be [T, K]")
    if rows is None:
        rows_a, nrows = None, M
    else:
        rows_a = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_a.shape[0]
    y = np.zeros((T, nrows), dtype=np.float64)
    A = np.zeros((T, nrows), dtype=np.float64)
    nt = nthreads or os.cpu_count() or 1
    _check(lib().qo_gemv(fmt, M, K, T, _ptr(codes), _ptr(scales), _ptr(x), _ptr(rows_a), nrows,
                         _ptr(y), _ptr(A), nt), "gemv")
    return y, A


def rtn_encode(bits: int, w: np.ndarray):
    """w: float64 [ngroups, 64] -> (codes int8 [ngroups, 64], scale bits uint16 [ngroups])."""
    w = np.ascontiguousarray(w, dtype=np.float64)
    n = w.shape[0]
    if w.shape != (n, 64):
        raise ValueError("w must be [ngroups, 64]")
    codes = np.empty((n, 64), dtype=np.int8)
    scales = np.empty((n,), dtype=np.uint16)
    _check(lib().qo_rtn_encode(bits, n, _ptr(w), _ptr(codes), _ptr(scales)), "rtn_encode")
    return codes, scales


def check(y: np.ndarray, y_ref: np.ndarray, A: np.ndarray, rel: float = REL_TOL, abs_: float = ABS_TOL):
    """Acceptance test for the product: |y - y_ref| <= rel * A + abs everywhere.
    Returns (ok, worst ratio |y - y_ref| / (rel*A + abs), index of the worst element)."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    bound = rel * A + abs_
    ratio = err / bound
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else ()
    wr = float(ratio[worst]) if ratio.size else 0.0
    return bool(wr <= 1.0), wr, worst


def logsumexp(y: np.ndarray) -> np.ndarray:
    """y: float [T, M] -> float64 [T]: log(sum_i exp(y[t, i])), evaluated as
    m + log(sum_i exp(y - m)) with m the row maximum (every term in (0, 1], no overflow)."""
    y = np.asarray(y, dtype=np.float64)
    if y.ndim != 2 or y.shape[1] == 0:
        raise ValueError("y must be [T, M] with M >= 1")
    m = y.max(axis=1)
    return m + np.log(np.exp(y - m[:, None]).sum(axis=1))


def topk(y: np.ndarray, k: int, index: Optional[np.ndarray] = None):
    """y: float [T, M] -> (values float64 [T, k], ids int64 [T, k]): per token the k largest
    values in descending order, equal values ordered by ascending row; ids are the rows, or
    index[row] when an index is given.  Slots past M hold -inf and id -1."""
    y = np.asarray(y, dtype=np.float64)
    T, M = y.shape
    vals = np.full((T, k), -np.inf)
    ids = np.full((T, k), -1, dtype=np.int64)
    rows = np.arange(M)
    for t in range(T):
        order = np.lexsort((rows, -y[t]))[:k]   # primary key -value, then row
        n = order.size
        vals[t, :n] = y[t, order]
        ids[t, :n] = order if index is None else np.asarray(index, dtype=np.int64)[order]
    return vals, ids


def grouped_search_encode(bits: int, w: np.ndarray, h: np.ndarray):
    """w, h: float64 [ngroups, 64] (h = per-channel importance of each group's columns)
    -> (codes int8 [ngroups, 64], scale bits uint16 [ngroups])."""
    w = np.ascontiguousarray(w, dtype=np.float64)
    h = np.ascontiguousarray(h, dtype=np.float64)
    n = w.shape[0]
    if w.shape != (n, 64) or h.shape != (n, 64):
        raise ValueError("w and h must be [ngroups, 64]")
    codes = np.empty((n, 64), dtype=np.int8)
    scales = np.empty((n,), dtype=np.uint16)
    _check(lib().qo_grouped_search_encode(bits, n, _ptr(w), _ptr(h), _ptr(codes), _ptr(scales)), "grouped_search")
    return codes, scales


def float_to_e4m3(q: float) -> int:
    return int(lib().qo_float_to_e4m3_rne_sat(float(q)))


def fp8_row_encode(w: np.ndarray):
    """w: float32 [M, K] -> (E4M3 bytes uint8 [M, K], row scales float32 [M])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    M, K = w.shape
    b = np.empty((M, K), dtype=np.uint8)
    r = np.empty((M,), dtype=np.float32)
    _check(lib().qo_fp8_row_encode(M, K, _ptr(w), _ptr(b), _ptr(r)), "fp8_row_encode")
    return b, r
