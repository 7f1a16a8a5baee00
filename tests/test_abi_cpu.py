"""The C ABI without a GPU: the library loads, exports every function include/qmat.h
declares with the binding's signature, and the host-side validation paths return the
documented status codes."""
import ctypes
import os
import re

import numpy as np
import pytest

import weight_only_quant_amd as wq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmat.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qmat_[a-z_]+)\s*\(", src)))


def test_header_lists_the_api():
    fns = header_functions()
    assert "qmat_run" in fns and "qmat_pack" in fns and len(fns) >= 9


def test_library_exports_every_header_function():
    L = ctypes.CDLL(wq.LIB_PATH)
    for name in header_functions():
        assert hasattr(L, name), name
    assert set(header_functions()) == set(wq.SIGNATURES)


def test_binding_loads():
    assert wq.lib() is not None


def _codes(fmt, M=64, K=128):
    if fmt == 8:
        return np.zeros((M, K), np.uint8), np.ones(M, np.float32)
    return np.zeros((M, K), np.int8), np.zeros((M, K // 64), np.uint16)


def _pack_raw(fmt, M, K, codes, scales, out_bytes=None):
    n = wq.qmat_packed_bytes(fmt, M, K) if out_bytes is None else out_bytes
    out = np.empty(max(n, 1), np.uint8)
    st = wq.lib().qmat_pack(fmt, M, K, codes.ctypes.data if codes is not None else None,
                            scales.ctypes.data if scales is not None else None, out.ctypes.data, n)
    return st


def test_binding_enum_values_match_the_header():
    # every QMAT_* enumerator of include/qmat.h has the same value in the binding
    import re
    text = open(os.path.join(ROOT, "include", "qmat.h")).read()
    found = dict((n, int(v)) for n, v in re.findall(r"\b(QMAT_[A-Z0-9_]+)\s*=\s*(-?\d+)", text))
    assert {"QMAT_ROUTE_MFMA_OFFSET", "QMAT_ROUTE_GEMM", "QMAT_Q8", "QMAT_ESIZE"} <= set(found)
    for name, value in found.items():
        if hasattr(wq, name):
            assert getattr(wq, name) == value, name
    assert wq.QMAT_ROUTE_MFMA_OFFSET == found["QMAT_ROUTE_MFMA_OFFSET"]


def test_packed_bytes_invalid_is_zero():
    assert wq.qmat_packed_bytes(3, 64, 128) == 0
    assert wq.qmat_packed_bytes(4, 0, 128) == 0
    assert wq.qmat_packed_bytes(4, 64, 100) == 0
    assert wq.qmat_packed_bytes(4, 64, 0) == 0
    assert wq.qmat_packed_bytes(4, 64, 64) > 0


def test_pack_errors():
    c, s = _codes(4)
    assert _pack_raw(7, 64, 128, c, s) == wq.QMAT_EINVAL
    assert _pack_raw(4, 64, 96, c, s) == wq.QMAT_ESHAPE
    assert _pack_raw(4, 0, 128, c, s) == wq.QMAT_ESHAPE
    assert _pack_raw(4, 64, 128, None, s) == wq.QMAT_EINVAL
    assert _pack_raw(4, 64, 128, c, s, out_bytes=100) == wq.QMAT_ESIZE
    assert "out_bytes" in wq.qmat_last_error()


@pytest.mark.parametrize("fmt,bad", [(4, 8), (4, -9), (5, 16), (5, -17), (6, 32), (6, -33)])
def test_pack_rejects_out_of_range_codes(fmt, bad):
    c, s = _codes(fmt)
    c[3, 77] = bad
    with pytest.raises(wq.QmatError) as e:
        wq.qmat_pack(fmt, c, s)
    assert e.value.status == wq.QMAT_ERANGE and "row 3 col 77" in str(e.value)


def test_pack_accepts_extreme_codes():
    for fmt, bits in ((4, 4), (5, 5), (6, 6), (wq.QMAT_Q8, 8)):
        c, s = _codes(fmt)
        c[0, 0], c[0, 1] = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
        wq.qmat_pack(fmt, c, s)


@pytest.mark.parametrize("bits", [0x7C00, 0xFC00, 0x7E00, 0x7C01])
def test_pack_rejects_nonfinite_half_scales(bits):
    c, s = _codes(4)
    s[5, 1] = bits
    with pytest.raises(wq.QmatError) as e:
        wq.qmat_pack(4, c, s)
    assert e.value.status == wq.QMAT_ERANGE


@pytest.mark.parametrize("byte", [0x7F, 0xFF])
def test_pack_rejects_nan_fp8(byte):
    c, s = _codes(8)
    c[2, 9] = byte
    with pytest.raises(wq.QmatError) as e:
        wq.qmat_pack(8, c, s)
    assert e.value.status == wq.QMAT_ERANGE


@pytest.mark.parametrize("val", [np.inf, -np.inf, np.nan])
def test_pack_rejects_nonfinite_row_scale(val):
    c, s = _codes(8)
    s[7] = val
    with pytest.raises(wq.QmatError) as e:
        wq.qmat_pack(8, c, s)
    assert e.value.status == wq.QMAT_ERANGE


def test_create_validation_without_gpu():
    L = wq.lib()
    h = ctypes.c_void_p()
    assert L.qmat_create(None, 4, 64, 128, 16, 100) == wq.QMAT_EINVAL
    assert L.qmat_create(ctypes.byref(h), 7, 64, 128, 16, 100) == wq.QMAT_EINVAL
    assert L.qmat_create(ctypes.byref(h), 4, 64, 100, 16, 100) == wq.QMAT_ESHAPE
    assert L.qmat_create(ctypes.byref(h), 4, 64, 128, None, 100) == wq.QMAT_EINVAL
    assert L.qmat_create(ctypes.byref(h), 4, 64, 128, 8, wq.qmat_packed_bytes(4, 64, 128)) == wq.QMAT_EINVAL  # misaligned
    assert L.qmat_create(ctypes.byref(h), 4, 64, 128, 16, 100) == wq.QMAT_ESIZE
    assert h.value is None


def test_create_view_rejects_null_arguments():
    L = wq.lib()
    h = ctypes.c_void_p()
    assert L.qmat_create_view(None, 16, 0, 64) == wq.QMAT_EINVAL
    assert L.qmat_create_view(ctypes.byref(h), None, 0, 64) == wq.QMAT_EINVAL
    assert h.value is None


def test_run_and_dequant_reject_null_handle():
    L = wq.lib()
    assert L.qmat_run(None, 16, 16, 1, None) == wq.QMAT_EINVAL
    assert L.qmat_run_ex(None, 16, 16, 1, 0, 0, 0, 0, None) == wq.QMAT_EINVAL
    assert L.qmat_dequant(None, 16, None) == wq.QMAT_EINVAL
    assert L.qmat_workspace_bytes(None, 0) == 0
    assert L.qmat_workspace_bytes(None, 1) == 0
    L.qmat_destroy(None)


PROBE_HEADER = os.path.join(ROOT, "include", "qmat_probe.h")


def test_probe_library_exports_its_header_and_validates():
    from weight_only_quant_amd import probe
    src = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(qmat_probe_[a-z_]+)\s*\(", src)))
    assert names == sorted(probe.SIGNATURES)
    L = probe.lib()
    for n in names:
        assert hasattr(L, n), n
    # out words: one per lane of every launched wave
    W = L.qmat_probe_read_out_words
    assert W(2048, 1, 4, 0) == 256              # 2 waves: one 4-wave workgroup
    assert W(1024 * 8, 2, 4, 0) == 256          # 4 waves: one
    assert W(1024 * 9, 2, 4, 0) == 2 * 256      # 5 waves: two
    assert W(1024 * 9, 2, 1, 0) == 5 * 64       # one-wave workgroups
    assert W(1024 * 9, 0, 8, 100) == 13 * 512   # grid-stride: 100 waves in 8-wave workgroups
    assert W(1024 * 9, 4, 4, -1) == 3 * 256     # workgroup runs of 4 chunks: 3 workgroups
    assert W(1024 * 9, 9, 2, -1) == 128         # one run
    for args in [(0, 1, 4, 0), (1000, 1, 4, 0), (1024, 0, 4, 0), (1024, 65537, 4, 0), (-1024, 1, 4, 0),
                 (1024, 1, 0, 0), (1024, 1, 9, 0), (1024, 1, 4, -2), (1024, 0, 4, -1),
                 (1024, 1, 4, (1 << 24) + 1)]:
        assert W(*args) == 0, args
    # host-side validation returns before any GPU call
    R = L.qmat_probe_read
    assert R(None, 1024, 1, 0, 1, 1, 0, 16, 64, None) == 1
    assert R(8, 1024, 1, 0, 1, 1, 0, 16, 64, None) == 1          # misaligned buffer
    assert R(16, 1000, 1, 0, 1, 1, 0, 16, 64, None) == 1         # not a multiple of 1 KB
    assert R(16, 1024, 1, 0, 3, 1, 0, 16, 64, None) == 1         # unroll
    assert R(16, 1024, 1, 0, 1, 1, 65537, 16, 64, None) == 1     # lds bytes
    assert R(16, 1024, 1, 0, 1, 9, 0, 16, 64 * 9, None) == 1     # waves per workgroup
    assert R(16, 1024, 1, 0, 1, 1, 0, None, 64, None) == 1       # null out
    assert R(16, 1024, 1, 0, 1, 1, 0, 16, 63, None) == 1         # out too small


def test_missing_library_fails_loudly():
    """With libqmat.so absent every binding call raises ImportError: there is no other path."""
    import subprocess
    import sys
    code = ("import weight_only_quant_amd as wq\n"
            "wq.LIB_PATH = '/nonexistent/libqmat.so'\n"
            "wq._lib = None\n"
            "try:\n"
            "    wq.qmat_packed_bytes(wq.QMAT_Q4, 64, 128)\n"
            "except ImportError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    print('no error')\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("raised:") and "no non-HIP path" in r.stdout, r.stdout


def test_product_code_never_uses_the_oracle():
    """The package (binding, build script, kernels, host sources) names no oracle module or
    oracle function: the oracle is test infrastructure only."""
    pkg = os.path.join(ROOT, "weight_only_quant_amd")
    offenders = []
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if not f.endswith((".py", ".hip", ".cpp", ".h")):
                continue
            src = open(os.path.join(dirpath, f), encoding="utf-8").read()
            if re.search(r"\bimport\s+oracle\b|\bfrom\s+oracle\b|\bqo_[a-z_0-9]+\s*\(|qmat_oracle", src):
                offenders.append(f)
    assert not offenders, offenders


def test_plan_struct_matches_header():
    """The binding's qmat_plan has the header's fields, in order, all int."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct\s*\{([^}]*)\}\s*qmat_plan;", src).group(1)
    fields = re.findall(r"\bint\s+([a-z_]+)\s*;", body)
    assert fields == [name for name, _ in wq.qmat_plan._fields_]
    assert all(t is ctypes.c_int for _, t in wq.qmat_plan._fields_)
    assert ctypes.sizeof(wq.qmat_plan) == 4 * len(fields)
