"""qmat_pack (host C++) against the documented layout, by round trip through the
independent numpy reader in layout_ref.py.  CPU only."""
import numpy as np
import pytest

import qmat_inputs as qi
import weight_only_quant_amd as wq
from layout_ref import dims, unpack

SHAPES = [(64, 128), (200, 320), (1, 64), (130, 192), (256, 1024)]


def _workload(fmt, M, K, seed):
    if fmt == 8:
        return qi.fp8_rows("t", M, K, 1, 0.01, seed)
    return qi.groupwise("t", fmt, M, K, 1, 0.01, seed)


@pytest.mark.parametrize("fmt", [4, 5, 6, 8, qi.Q8])
@pytest.mark.parametrize("M,K", SHAPES)
def test_pack_round_trip(fmt, M, K):
    wl = _workload(fmt, M, K, M + K + fmt)
    blob = wq.qmat_pack(fmt, wl.codes, wl.scales)
    NT, NU, cb, sb = dims(fmt, M, K)
    assert blob.size == cb + sb == wq.qmat_packed_bytes(fmt, M, K)
    codes, scales, full_codes, full_scales = unpack(fmt, M, K, blob)
    assert np.array_equal(codes, wl.codes)
    if fmt == 8:
        assert np.array_equal(scales.view(np.uint32), wl.scales.view(np.uint32))
    else:
        assert np.array_equal(scales, wl.scales)
    # padding rows / columns / groups are zero
    pad = full_codes.copy()
    pad[:M, :K] = 0
    assert not pad.any()
    sp = full_scales.copy()
    if fmt == 8:
        sp[:M] = 0
    else:
        sp[:M, :K // 64] = 0
    assert not sp.any()


@pytest.mark.parametrize("fmt", [4, 5, 6, qi.Q8])
def test_pack_every_code_at_every_position(fmt):
    # each code value visits every position of every k octet and every row slot of a tile
    bits = qi.code_bits(fmt)
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    n = hi - lo + 1
    M, K = 64 + 5, 256
    r = np.arange(M)[:, None]
    k = np.arange(K)[None, :]
    codes = (lo + (r * 7 + k * 3 + (k // 8) * 5) % n).astype(np.int8)
    scales = (np.arange(M * (K // 64), dtype=np.uint16).reshape(M, K // 64) * 37) & np.uint16(0x7BFF)
    blob = wq.qmat_pack(fmt, codes, scales)
    c2, s2, _, _ = unpack(fmt, M, K, blob)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


def test_pack_fp8_every_byte():
    byts = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    M, K = 3, 256
    codes = np.resize(byts, (M, K)).astype(np.uint8)
    rs = np.array([1.5, -2.0, 1e-30], np.float32)
    blob = wq.qmat_pack(8, codes, rs)
    c2, s2, _, _ = unpack(8, M, K, blob)
    assert np.array_equal(c2, codes) and np.array_equal(s2, rs)


def test_packed_bytes_per_weight():
    # 0.5 / 0.625 / 0.75 / 1 bytes per weight, plus 2 bytes per 64-group (4 per FP8 row)
    M, K = 34816, 5120
    assert wq.qmat_packed_bytes(4, M, K) == M * K // 2 + M * (K // 64) * 2
    assert wq.qmat_packed_bytes(5, 5120, 17408) == 5120 * 17408 * 5 // 8 + 5120 * 272 * 2
    assert wq.qmat_packed_bytes(6, 248320, 5120) == 248320 * 5120 * 3 // 4 + 248320 * 80 * 2
    assert wq.qmat_packed_bytes(8, 248320, 5120) == 248320 * 5120 + 248320 * 4
    assert wq.qmat_packed_bytes(wq.QMAT_Q8, 248320, 5120) == 248320 * 5120 + 248320 * 80 * 2
