"""Pins for the CPU oracle against facts fixed outside it.

Each test checks an oracle function against something the oracle does not compute
itself: a library's independent implementation (numpy / torch conversions, numpy
float64 matmul), exact rational arithmetic (fractions), closed forms, hand-worked
cases (tests/golden/), or invariants of the definition.  A plausible slip in the
oracle (a wrong exponent bias, a dropped subnormal branch, a sign error, a
transposed operand, a missing group index) fails at least one of them; the
comments name which.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import qmat_inputs as qi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _same_float(a: float, b: float) -> bool:
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


# ------------------------------------------------------------------ decoders

def test_half_decoder_every_pattern():
    # library cross-check: numpy's binary16 -> float64 conversion (catches a wrong
    # bias, a missing subnormal branch, inf/NaN handling, the sign of zero)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    nan_ref, nan_got = np.isnan(ref), np.isnan(got)
    assert np.array_equal(nan_ref, nan_got)
    m = ~nan_ref
    assert np.array_equal(got[m], ref[m])
    assert np.array_equal(np.signbit(got[m]), np.signbit(ref[m]))


def test_bf16_decoder_every_pattern():
    # library cross-check: torch bfloat16 -> float64
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_double(int(b) & 0xFFFF) for b in bits.numpy()])
    nan_ref, nan_got = np.isnan(ref), np.isnan(got)
    assert np.array_equal(nan_ref, nan_got)
    m = ~nan_ref
    assert np.array_equal(got[m], ref[m])
    assert np.array_equal(np.signbit(got[m]), np.signbit(ref[m]))


def test_e4m3_decoder_every_byte_vs_torch():
    # library cross-check: torch.float8_e4m3fn is the OCP E4M3 ("FN") format
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_to_double(b) for b in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m])
    assert np.array_equal(np.signbit(got[m]), np.signbit(ref[m]))
    assert np.isnan(got).sum() == 2  # only 0x7F and 0xFF


def _parse_val(s: str) -> float:
    s = s.strip()
    if s == "nan":
        return float("nan")
    if s == "-0":
        return -0.0
    if "2^" in s:
        coef, _, exp = s.partition("2^")
        coef = coef.rstrip("*")
        return (float(coef) if coef else 1.0) * 2.0 ** int(exp)
    return float(s)


def test_e4m3_decoder_spec_table():
    # golden values of the OCP spec (max 448, min normal 2^-6, min subnormal 2^-9)
    spec = json.load(open(os.path.join(GOLDEN, "e4m3_ocp_spot.json")))
    for byte, val in spec["values"]:
        assert _same_float(oracle.e4m3_to_double(int(byte, 16)), _parse_val(val)), byte


def test_double_to_half_matches_numpy_rne():
    # library cross-check of the encoder's rounding: numpy rounds float64 -> float16
    # correctly (nearest, ties to even).  Includes exact ties, the subnormal range,
    # the overflow threshold and values that carry into the next binade.
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(20000) * np.exp(rng.uniform(-25, 12, 20000)))
    for e in range(-26, 17):
        base = 2.0 ** e
        for k in range(0, 2049, 7):
            vals.append(base * (1 + k / 2048.0))  # includes half-quantum ties
            vals.append(-base * (1 + (k + 0.5) / 2048.0))
    vals += [0.0, -0.0, 65504.0, 65519.99, 65520.0, 70000.0, 2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25,
             2.0 ** -26, 2.0 ** -14 - 2.0 ** -25, 1 - 2.0 ** -12, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11]
    arr = np.array(vals, dtype=np.float64)
    with np.errstate(over="ignore"):
        ref = arr.astype(np.float16).view(np.uint16)
    got = np.array([oracle.double_to_half(v) for v in arr], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(arr[i], hex(got[i]), hex(ref[i])) for i in bad[:5]]


# ------------------------------------------------------------------ dequant

SCALE_SET = [0.0, -0.0, 2.0 ** -24, -(2.0 ** -24), 2.0 ** -14 - 2.0 ** -24, -(2.0 ** -14 - 2.0 ** -24),
             2.0 ** -14, -(2.0 ** -14), 1.0, -1.0, 65504.0, -65504.0, 0.3333, -7.125, 1e-3]


@pytest.mark.parametrize("bits", [4, 5, 6, 8])
def test_dequant_every_code_times_every_scale_is_exact(bits):
    # brute force: each code value at each position of a group, times scales that
    # include signed zeros, subnormals, the largest normal; the result must be the
    # exact rational product with the IEEE sign of zero (catches a scale taken from
    # the wrong group, code sign errors, rounding, -0 handling)
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    codes_1d = np.arange(lo, hi + 1, dtype=np.int8)
    n = codes_1d.size
    sbits = np.array(SCALE_SET, dtype=np.float16).view(np.uint16)
    G = len(sbits)
    K = 64 * G
    # row r puts code (r + j) mod n at position j of each group, so every code
    # value visits every position, under every scale
    M = n
    codes = np.empty((M, K), dtype=np.int8)
    for r in range(M):
        codes[r] = codes_1d[(r + np.arange(K)) % n]
    scales = np.tile(sbits, (M, 1))
    w = oracle.dequant_groupwise(bits, codes, scales)
    for r in range(M):
        for j in range(K):
            s = float(np.uint16(scales[r, j // 64]).view(np.float16))
            exact = Fraction(s) * int(codes[r, j])
            got = float(w[r, j])
            assert Fraction(got) == exact, (r, j)
            if exact == 0:
                want_neg = (math.copysign(1, s) < 0) != (codes[r, j] < 0)
                assert (math.copysign(1, got) < 0) == want_neg, (r, j, s, codes[r, j])


def test_gemv_q8_is_the_groupwise_definition_with_8_bit_codes():
    # format id 9 (8-bit groupwise) gives exactly what the groupwise dequant with 8-bit
    # codes gives; an 8-bit code matrix whose codes fit in 6 bits gives the Q6 result
    wl = qi.groupwise("t", qi.Q8, 19, 192, 2, 0.01, 4)
    y8, A8 = oracle.gemv(qi.Q8, wl.codes, wl.scales, wl.x)
    W = oracle.dequant_groupwise(8, wl.codes, wl.scales).astype(np.float64)
    X = _x64(wl.x)
    assert np.all(np.abs(y8 - X @ W.T) <= 1e-12 * A8)
    small = np.clip(wl.codes, -32, 31).astype(np.int8)
    y8s, _ = oracle.gemv(qi.Q8, small, wl.scales, wl.x)
    y6, _ = oracle.gemv(6, small, wl.scales, wl.x)
    assert np.array_equal(y8s, y6)


def test_dequant_rejects_out_of_range_codes():
    codes = np.zeros((1, 64), dtype=np.int8)
    codes[0, 5] = 8
    with pytest.raises(oracle.OracleError):
        oracle.dequant_groupwise(4, codes, np.zeros((1, 1), dtype=np.uint16))
    codes[0, 5] = -17
    with pytest.raises(oracle.OracleError):
        oracle.dequant_groupwise(5, codes, np.zeros((1, 1), dtype=np.uint16))


def test_dequant_fp8_every_byte_is_one_rounded_product():
    # each finite byte times row scales (normal, tiny, huge, negative); the result
    # must be the fp32 nearest-even rounding of the exact product: numpy's float32
    # multiply of the two (exactly representable) factors is that rounding
    byts = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    rs = np.array([1.0, 0.0123, 3.0e-5, 1.7e-38, 1e-40, 2.5e30, -0.75, 7.0 / 3.0], dtype=np.float32)
    M = rs.size
    b2 = np.tile(byts, (M, 1))
    pad = (-b2.shape[1]) % 64
    b2 = np.concatenate([b2, np.zeros((M, pad), np.uint8)], axis=1)
    w = oracle.dequant_fp8(b2, rs)
    dec = torch.from_numpy(b2.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    with np.errstate(over="ignore", under="ignore"):
        ref = rs[:, None] * dec
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))


def test_dequant_fp8_rejects_nan_bytes():
    b = np.zeros((1, 64), np.uint8)
    b[0, 3] = 0xFF
    with pytest.raises(oracle.OracleError):
        oracle.dequant_fp8(b, np.ones(1, np.float32))


def test_golden_worked_dequant_cases():
    spec = json.load(open(os.path.join(GOLDEN, "groupwise_worked.json")))
    case = next(c for c in spec["cases"] if c["name"] == "negative_scale_reaches_min_code")
    for code, sb, val in case["dequant"]:
        codes = np.zeros((1, 64), np.int8)
        codes[0, 0] = code
        w = oracle.dequant_groupwise(case["bits"], codes, np.array([[int(sb, 16)]], np.uint16))
        assert _same_float(float(w[0, 0]), float(val)), (code, sb, val, w[0, 0])


# ------------------------------------------------------------------ product

def _small_groupwise(bits, M, K, T, seed):
    return qi.groupwise("t", bits, M, K, T, 0.01, seed)


def _exact_w64(wl):
    """float64 dequant built from library conversions (numpy fp16, torch e4m3) —
    independent of the oracle's decoders."""
    if wl.fmt == 8:
        dec = torch.from_numpy(wl.codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        return wl.scales.astype(np.float64)[:, None] * dec
    s = wl.scales.view(np.float16).astype(np.float64)
    return np.repeat(s, 64, axis=1) * wl.codes.astype(np.float64)


def _x64(x_bits):
    return torch.from_numpy(x_bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("fmt", [4, 5, 6, 8, qi.Q8])
def test_gemv_matches_float64_matmul(fmt):
    # library cross-check: numpy float64 matmul on an independently dequantized
    # matrix (catches a transposed operand, a wrong group index, a scale applied
    # per row instead of per group, a dropped term)
    M, K, T = 37, 320, 3
    wl = qi.fp8_rows("t", M, K, T, 0.01, 3) if fmt == 8 else _small_groupwise(fmt, M, K, T, 3)
    y, A = oracle.gemv(fmt, wl.codes, wl.scales, wl.x)
    W = _exact_w64(wl)
    X = _x64(wl.x)
    y_ref = X @ W.T
    A_ref = np.abs(X) @ np.abs(W).T
    assert np.all(np.abs(y - y_ref) <= 1e-12 * A_ref + 1e-300)
    assert np.allclose(A, A_ref, rtol=1e-12, atol=0)


@pytest.mark.parametrize("fmt", [4, 6, 8, qi.Q8])
def test_gemv_brute_force_exact_fractions(fmt):
    # exact rational sum on a tiny case; the oracle may differ only by its double
    # summation error (<= K * 2^-53 * A)
    M, K, T = 3, 128, 2
    wl = qi.fp8_rows("t", M, K, T, 0.01, 5) if fmt == 8 else _small_groupwise(fmt, M, K, T, 5)
    y, A = oracle.gemv(fmt, wl.codes, wl.scales, wl.x)
    W = _exact_w64(wl)
    X = _x64(wl.x)
    for t in range(T):
        for i in range(M):
            exact = sum(Fraction(float(W[i, j])) * Fraction(float(X[t, j])) for j in range(K))
            assert abs(Fraction(float(y[t, i])) - exact) <= Fraction(K) * Fraction(2) ** -53 * Fraction(float(A[t, i]))


def test_gemv_one_hot_returns_column():
    # x = e_j selects column j of W exactly
    wl = _small_groupwise(5, 20, 192, 1, 7)
    W = oracle.dequant_groupwise(5, wl.codes, wl.scales)
    for j in [0, 63, 64, 100, 191]:
        x = np.zeros((1, 192), np.uint16)
        x[0, j] = 0x3F80  # bf16 1.0
        y, _ = oracle.gemv(5, wl.codes, wl.scales, x)
        assert np.array_equal(y[0], W[:, j].astype(np.float64))


def test_gemv_linearity_and_identical_tokens():
    wl = _small_groupwise(4, 30, 256, 1, 8)
    x2 = (wl.x.astype(np.uint32) + (1 << 7)).astype(np.uint16)  # exponent + 1: exactly 2x (no zero/inf here)
    assert not np.any((wl.x & 0x7F80) == 0)
    xx = np.concatenate([wl.x, x2, wl.x], axis=0)
    y, A = oracle.gemv(4, wl.codes, wl.scales, xx)
    assert np.array_equal(y[1], 2 * y[0])
    assert np.array_equal(y[2], y[0]) and np.array_equal(A[2], A[0])
    neg = wl.x ^ np.uint16(0x8000)
    yn, _ = oracle.gemv(4, wl.codes, wl.scales, neg)
    assert np.array_equal(yn[0], -y[0])


def test_gemv_row_subset_matches_full():
    wl = _small_groupwise(6, 50, 128, 2, 9)
    y, A = oracle.gemv(6, wl.codes, wl.scales, wl.x)
    rows = [49, 0, 17, 17, 3]
    ys, As = oracle.gemv(6, wl.codes, wl.scales, wl.x, rows=rows, nthreads=3)
    assert np.array_equal(ys, y[:, rows]) and np.array_equal(As, A[:, rows])


def test_gemv_golden_product():
    spec = json.load(open(os.path.join(GOLDEN, "groupwise_worked.json")))
    case = next(c for c in spec["cases"] if c["name"] == "product_ones")
    j = np.arange(64)
    codes = ((j % 16) - 8).astype(np.int8)[None, :]
    scales = np.array([[0x3800]], np.uint16)
    x = np.full((1, 64), 0x3F80, np.uint16)
    y, A = oracle.gemv(4, codes, scales, x)
    assert y[0, 0] == float(case["y"]) and A[0, 0] == float(case["A"])


# ------------------------------------------------------------------ encoder

def _eval_expr(expr, j):
    return eval(expr, {"__builtins__": {}}, {"j": j})  # expressions from the golden file


def test_rtn_golden_cases():
    spec = json.load(open(os.path.join(GOLDEN, "groupwise_worked.json")))
    for case in spec["cases"]:
        if "w" not in case:
            continue
        w = np.array([[_eval_expr(case["w"], j) for j in range(64)]], dtype=np.float64)
        codes, sb = oracle.rtn_encode(case["bits"], w)
        assert int(sb[0]) == int(case["scale_bits"], 16), case["name"]
        assert codes[0].tolist() == [_eval_expr(case["codes"], j) for j in range(64)], case["name"]


@pytest.mark.parametrize("bits", [4, 5, 6, 8])
def test_rtn_invariants(bits):
    rng = np.random.default_rng(bits)
    n = 400
    w = rng.standard_normal((n, 64)) * np.exp(rng.uniform(-8, 4, (n, 1)))
    w[0] = 0.0
    codes, sb = oracle.rtn_encode(bits, w)
    qmax, qmin = (1 << (bits - 1)) - 1, -(1 << (bits - 1))
    s = sb.view(np.float16).astype(np.float64)
    assert codes.min() >= qmin and codes.max() <= qmax
    assert sb[0] == 0 and np.all(codes[0] == 0)
    # RTN never produces negative scales or the most negative code
    assert np.all(s >= 0) and codes.min() > qmin
    # the stored scale is the nearest FP16 to absmax/qmax
    a = np.abs(w).max(axis=1)
    assert np.array_equal(sb, (a / qmax).astype(np.float16).view(np.uint16))
    # reconstruction error is at most half a step unless the code was clamped
    err = np.abs(w - s[:, None] * codes)
    clamped = np.abs(codes) == qmax
    assert np.all((err <= s[:, None] / 2 * (1 + 1e-12)) | clamped)
    # the group's absmax element maps to +-qmax (fp16 rounding of the scale moves
    # w/s by less than 2^-11 * qmax, so it still rounds or clamps to qmax)
    idx = np.abs(w[1:]).argmax(axis=1)
    assert np.all(np.abs(codes[1:][np.arange(n - 1), idx]) == qmax)


def test_rtn_power_of_two_scale_round_trip():
    # a group built as s*c with s a power of two and a code hitting +-qmax returns (s, c)
    rng = np.random.default_rng(0)
    for bits in (4, 5, 6, 8):
        qmax = (1 << (bits - 1)) - 1
        for e in range(-20, 10):
            c = rng.integers(-qmax, qmax + 1, 64)
            c[rng.integers(64)] = qmax * (1 if rng.random() < 0.5 else -1)
            s = 2.0 ** e
            codes, sb = oracle.rtn_encode(bits, (s * c)[None, :].astype(np.float64))
            assert np.array_equal(codes[0], c) and float(np.uint16(sb[0]).view(np.float16)) == s


def test_rtn_rejects_overflow():
    with pytest.raises(oracle.OracleError):
        oracle.rtn_encode(4, np.full((1, 64), 1e6))


# ------------------------------------------------------------------ acceptance test

def test_check_flags_errors_beyond_tolerance():
    y_ref = np.array([[1.0, -2.0, 0.0]])
    A = np.array([[10.0, 5.0, 0.0]])
    ok, r, _ = oracle.check(y_ref + np.array([[9e-4, -4e-4, 9e-7]]), y_ref, A)
    assert ok and r < 1
    ok, r, idx = oracle.check(y_ref + np.array([[0.0, 0.0, 2e-6]]), y_ref, A)
    assert not ok and idx == (0, 2)
    ok, _, _ = oracle.check(np.array([[np.nan, -2.0, 0.0]]), y_ref, A)
    assert not ok


# ------------------------------------------------------------------ head epilogue: log-sum-exp and top-k

def test_logsumexp_closed_forms():
    # a constant row: c + log M exactly; one dominant value: that value (the rest underflow
    # relative to it); duplicating every value adds log 2
    for M in (1, 7, 64, 1000):
        for c in (0.0, -3.5, 41.0, 1e-3):
            got = oracle.logsumexp(np.full((1, M), c))
            assert abs(got[0] - (c + math.log(M))) <= 1e-15 * max(1.0, abs(c) + math.log(M))
    y = np.array([[1000.0, 0.0, -5.0, 3.0]])
    assert oracle.logsumexp(y)[0] == 1000.0
    rng = np.random.default_rng(2)
    z = rng.standard_normal((3, 77)) * 4
    assert np.allclose(oracle.logsumexp(np.concatenate([z, z], axis=1)), oracle.logsumexp(z) + math.log(2),
                       rtol=0, atol=1e-13)


def test_logsumexp_matches_scipy_and_is_shift_equivariant():
    # library cross-check (scipy.special.logsumexp), bounds max <= lse <= max + log M, and
    # lse(y + c) = lse(y) + c
    from scipy.special import logsumexp as sp_lse
    y = qi.logits(5, 3000, 7).astype(np.float64)
    got = oracle.logsumexp(y)
    assert np.allclose(got, sp_lse(y, axis=1), rtol=0, atol=1e-12)
    mx = y.max(axis=1)
    assert np.all(got >= mx) and np.all(got <= mx + math.log(y.shape[1]))
    assert np.allclose(oracle.logsumexp(y + 17.25), got + 17.25, rtol=0, atol=1e-12)


def test_topk_brute_force_with_ties_and_index():
    # brute force: Python's sort by (value descending, row ascending) on tiny rows full of
    # ties, with and without an index map; k beyond M pads with (-inf, -1)
    rng = np.random.default_rng(3)
    for trial in range(40):
        M = int(rng.integers(1, 40))
        T = int(rng.integers(1, 4))
        y = rng.integers(-3, 4, (T, M)).astype(np.float32) * 0.5
        index = rng.permutation(10 * M)[:M] if trial % 2 else None
        for k in (1, 3, 8, 45):
            vals, ids = oracle.topk(y, k, index)
            for t in range(T):
                want = sorted(range(M), key=lambda r: (-float(y[t, r]), r))[:k]
                n = len(want)
                assert vals[t, :n].tolist() == [float(y[t, r]) for r in want]
                assert ids[t, :n].tolist() == [int(index[r]) if index is not None else r for r in want]
                assert np.all(vals[t, n:] == -np.inf) and np.all(ids[t, n:] == -1)


def test_logits_generator_plants_ties():
    y = qi.logits(4, 5000, 9)
    for t in range(4):
        assert np.sum(y[t] == y[t].max()) >= 2


# ------------------------------------------------------------------ encoders

def test_e4m3_encoder_round_trips_and_matches_torch():
    # every finite E4M3 value encodes to its own byte; a dense sweep of in-range floats
    # (|q| < 464, where torch's nearest-even conversion does not produce NaN) matches torch;
    # beyond 448 the encoder saturates
    for b in range(256):
        if (b & 0x7F) == 0x7F:
            continue
        v = oracle.e4m3_to_double(b)
        assert oracle.float_to_e4m3(v) == b, hex(b)
    rng = np.random.default_rng(0)
    q = np.concatenate([rng.uniform(-463.9, 463.9, 20000), rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 6, 20000),
                        (np.arange(-2000, 2001) * 2.0 ** -10)]).astype(np.float32)
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.float_to_e4m3(float(v)) for v in q], np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(q[i], hex(got[i]), hex(ref[i])) for i in bad[:5]]
    for v, b in [(448.0, 0x7E), (463.9, 0x7E), (470.0, 0x7E), (1e30, 0x7E), (-5000.0, 0xFE), (-0.0, 0x80)]:
        assert oracle.float_to_e4m3(v) == b, v


def test_fp8_row_encode_properties():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((40, 192)) * np.exp(rng.uniform(-6, 3, (40, 1)))).astype(np.float32)
    w[3] = 0.0
    b, r = oracle.fp8_row_encode(w)
    assert r[3] == 0 and np.all(b[3] == 0)
    dec = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    a = np.abs(w).max(axis=1)
    assert np.array_equal(r, (a.astype(np.float64) / 448.0).astype(np.float32))
    for i in range(40):
        if a[i] == 0:
            continue
        # the row's largest magnitude lands on +-448; every value is within half an E4M3
        # quantum (relative 2^-4, or 2^-10 absolute among subnormals) of w / r
        j = int(np.abs(w[i]).argmax())
        assert abs(dec[i, j]) == 448.0
        q = (w[i] / r[i]).astype(np.float64)
        assert np.all(np.abs(dec[i] - q) <= np.maximum(np.abs(q) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-9))


def _gs_error(w, h, s, c):
    return float(np.sum(h * (w - s * c) ** 2))


def test_grouped_search_golden_case():
    spec = json.load(open(os.path.join(GOLDEN, "grouped_search_worked.json")))
    for case in spec["cases"]:
        w = np.zeros((1, 64))
        w[0, :len(case["w_head"])] = case["w_head"]
        h = np.ones((1, 64))
        codes, sb = oracle.grouped_search_encode(case["bits"], w, h)
        assert int(sb[0]) == int(case["scale_bits"], 16)
        assert codes[0, :3].tolist() == case["codes_head"] and not codes[0, 3:].any()
        rc, rsb = oracle.rtn_encode(case["bits"], w)
        assert int(rsb[0]) == int(case["rtn_scale_bits"], 16) and rc[0, :3].tolist() == case["rtn_codes_head"]
        rs = float(np.uint16(rsb[0]).view(np.float16))
        assert abs(_gs_error(w[0], h[0], rs, rc[0]) - case["rtn_error"]) < 1e-7


@pytest.mark.parametrize("bits", [4, 5, 6, 8])
def test_grouped_search_is_the_best_candidate_and_never_worse_than_rtn(bits):
    # brute force over the 50 candidates with numpy's float16 rounding: the chosen scale has
    # the smallest weighted error (first of equals); RTN's scale is candidate 0, so the search
    # is never worse than RTN; codes stay in range; some groups choose negative scales
    rng = np.random.default_rng(bits)
    n = 120
    w = rng.standard_normal((n, 64)) * np.exp(rng.uniform(-5, 2, (n, 1)))
    w[0] = 0.0
    h = rng.exponential(1.0, (n, 64)) * (rng.random((n, 64)) < 0.9)
    codes, sb = oracle.grouped_search_encode(bits, w, h)
    rc, rsb = oracle.rtn_encode(bits, w)
    qmax, qmin = (1 << (bits - 1)) - 1, -(1 << (bits - 1))
    assert codes.min() >= qmin and codes.max() <= qmax
    assert sb[0] == 0 and not codes[0].any()
    s = sb.view(np.float16).astype(np.float64)
    negs = 0
    for g in range(1, n):
        a = np.abs(w[g]).max()
        errs = []
        for cand in range(50):
            i = cand // 2
            mag = a / (qmax + i / 24.0)
            sc = float(np.float16(-mag if cand % 2 else mag))
            c = np.clip(np.rint(w[g] / sc), qmin, qmax) if sc != 0 else np.zeros(64)
            errs.append(_gs_error(w[g], h[g], sc, c))
        best = int(np.argmin(errs))
        assert s[g] == float(np.float16(-(a / (qmax + (best // 2) / 24.0)) if best % 2 else a / (qmax + (best // 2) / 24.0)))
        assert _gs_error(w[g], h[g], s[g], codes[g]) == errs[best]
        rs = float(np.uint16(rsb[g]).view(np.float16))
        assert errs[best] <= _gs_error(w[g], h[g], rs, rc[g])
        negs += s[g] < 0
    assert negs > 0


def test_grouped_search_recovers_full_range_groups_exactly():
    # a group s*c whose codes use -2^(b-1), with s a power of two: the negative-sign candidate
    # -a/2^(b-1) reproduces it with zero error (RTN cannot)
    rng = np.random.default_rng(7)
    for bits in (4, 5, 6, 8):
        qmax, qmin = (1 << (bits - 1)) - 1, -(1 << (bits - 1))
        for e in (-12, -3, 0, 4):
            c = rng.integers(qmin + 1, qmax + 1, 64)
            c[rng.integers(64)] = qmin
            sgn = 1 if rng.random() < 0.5 else -1
            w = (sgn * 2.0 ** e * c)[None, :].astype(np.float64)
            codes, sb = oracle.grouped_search_encode(bits, w, np.ones((1, 64)))
            s = float(np.uint16(sb[0]).view(np.float16))
            assert _gs_error(w[0], np.ones(64), s, codes[0]) == 0.0
            assert np.array_equal(s * codes[0].astype(np.float64), w[0])
