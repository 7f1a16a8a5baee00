"""qmat_quantize (the library's host encoders) against the oracle's encoders, bit for bit:
upstream RTN and the grouped search for Q4/Q5/Q6/Q8, and the row-scaled FP8 encoder.  The two
sides share no code (the library uses the compiler's binary16 conversions and a bit-level E4M3
rounding; the oracle its own decoders and frexp-based rounding).  CPU only."""
import numpy as np
import pytest

import oracle
import qmat_inputs as qi
import weight_only_quant_amd as wq


def _weights(M, K, seed):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((M, K)) * np.exp(rng.uniform(-7, 3, (M, 1)))
    w[0] = 0.0                                    # an all-zero row
    w[1, :64] = 0.0                               # an all-zero group
    w[2, 5] = -np.abs(w[2]).max() * 3             # a negative group maximum
    w[3, 64:128] = np.round(w[3, 64:128] * 4) / 4  # many exact ties in w / s
    return w.astype(np.float32)


def _groups(w):
    M, K = w.shape
    return w.astype(np.float64).reshape(M * (K // 64), 64)


@pytest.mark.parametrize("fmt", [4, 5, 6, qi.Q8])
def test_rtn_matches_oracle(fmt):
    w = _weights(37, 320, fmt)
    codes, scales = wq.qmat_quantize(fmt, w, encoder=wq.QMAT_ENCODE_RTN)
    oc, os_ = oracle.rtn_encode(qi.code_bits(fmt), _groups(w))
    assert np.array_equal(codes.reshape(-1, 64), oc) and np.array_equal(scales.reshape(-1), os_)


@pytest.mark.parametrize("fmt", [4, 5, 6, qi.Q8])
@pytest.mark.parametrize("with_importance", [False, True])
def test_grouped_search_matches_oracle(fmt, with_importance):
    M, K = 29, 384
    w = _weights(M, K, 10 + fmt)
    rng = np.random.default_rng(fmt)
    imp = (rng.exponential(1.0, K) * (rng.random(K) < 0.85)).astype(np.float32) if with_importance else None
    codes, scales = wq.qmat_quantize(fmt, w, imp, encoder=wq.QMAT_ENCODE_GROUPED_SEARCH)
    h = np.tile(imp.astype(np.float64) if imp is not None else np.ones(K), (M, 1)).reshape(-1, 64)
    oc, os_ = oracle.grouped_search_encode(qi.code_bits(fmt), _groups(w), h)
    assert np.array_equal(codes.reshape(-1, 64), oc)
    assert np.array_equal(scales.reshape(-1), os_)
    assert np.any(scales.view(np.int16) < 0)  # some groups take negative scales


def test_fp8_row_encoder_matches_oracle():
    w = _weights(41, 256, 3)
    w[4, 7] = 1e-42   # an fp32 subnormal weight
    b, r = wq.qmat_quantize(wq.QMAT_FP8_E4M3_ROW, w)
    ob, orr = oracle.fp8_row_encode(w)
    assert np.array_equal(b, ob) and np.array_equal(r.view(np.uint32), orr.view(np.uint32))


def test_quantize_then_pack_round_trips():
    # the encoder's output is a valid qmat_pack input
    w = _weights(70, 192, 5)
    for fmt in (4, 5, 6, qi.Q8, 8):
        enc = wq.QMAT_ENCODE_RTN if fmt == 8 else wq.QMAT_ENCODE_GROUPED_SEARCH
        codes, scales = wq.qmat_quantize(fmt, w, encoder=enc)
        blob = wq.qmat_pack(fmt, codes, scales)
        assert blob.size == wq.qmat_packed_bytes(fmt, 70, 192)


def test_quantize_errors():
    w = np.ones((4, 64), np.float32)
    L = wq.lib()
    c, s = np.empty((4, 64), np.int8), np.empty((4, 1), np.uint16)
    assert L.qmat_quantize(7, 4, 64, w.ctypes.data, None, 0, c.ctypes.data, s.ctypes.data) == wq.QMAT_EINVAL
    assert L.qmat_quantize(4, 4, 64, w.ctypes.data, None, 2, c.ctypes.data, s.ctypes.data) == wq.QMAT_EINVAL
    assert L.qmat_quantize(4, 4, 100, w.ctypes.data, None, 0, c.ctypes.data, s.ctypes.data) == wq.QMAT_ESHAPE
    assert L.qmat_quantize(4, 4, 64, None, None, 0, c.ctypes.data, s.ctypes.data) == wq.QMAT_EINVAL
    assert L.qmat_quantize(8, 4, 64, w.ctypes.data, None, 1, c.ctypes.data, s.ctypes.data) == wq.QMAT_EINVAL
    bad = w.copy()
    bad[2, 3] = np.nan
    with pytest.raises(wq.QmatError) as e:
        wq.qmat_quantize(4, bad)
    assert e.value.status == wq.QMAT_ERANGE
    with pytest.raises(wq.QmatError) as e:
        wq.qmat_quantize(4, np.full((1, 64), 1e6, np.float32))  # 1e6 / 7 overflows FP16
    assert e.value.status == wq.QMAT_ERANGE
    with pytest.raises(wq.QmatError) as e:
        wq.qmat_quantize(4, w, -np.ones(64, np.float32), encoder=wq.QMAT_ENCODE_GROUPED_SEARCH)
    assert e.value.status == wq.QMAT_ERANGE
