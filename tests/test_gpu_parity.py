"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

  - qmat_dequant must equal the oracle's dequantization bit for bit (sign of zero included);
  - qmat_run must satisfy |y - y_ref| <= 1e-4 * sum_j |w_ij x_tj| + 1e-6 everywhere, and match
    bit for bit on inputs where every partial sum is exact in fp32.
Small shapes span several 64-row tiles with a ragged last tile and odd group counts; the full
benchmark shapes are checked on every row in the launch configuration the benchmark uses.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import qmat_inputs as qi
import weight_only_quant_amd as wq

pytestmark = pytest.mark.gpu

ROUTES = {"valu": wq.QMAT_ROUTE_VALU, "mfma": wq.QMAT_ROUTE_MFMA}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    wq.lib()
    return torch.device("cuda:0")


def _workload(fmt, M, K, T, seed, mult=0.01):
    if fmt == 8:
        return qi.fp8_rows("t", M, K, T, mult, seed)
    return qi.groupwise("t", fmt, M, K, T, mult, seed)


def _x_dev(x_bits):
    return torch.from_numpy(x_bits.view(np.int16).copy()).view(torch.bfloat16).cuda()


def _check_y(y, wl, label, rows=None):
    y_ref, A = oracle.gemv(wl.fmt, wl.codes, wl.scales, wl.x, rows=rows)
    got = y.detach().cpu().numpy().astype(np.float64)
    if rows is not None:
        got = got[:, rows]
    ok, worst, idx = oracle.check(got, y_ref, A)
    assert ok, f"{label}: worst |err|/(1e-4*A+1e-6) = {worst:.3g} at {idx}: got {got[idx]!r} want {y_ref[idx]!r} A {A[idx]!r}"
    return worst


# ------------------------------------------------------------------ dequant: bit exact

DQ_SHAPES = [(64, 128), (200, 320), (1, 64), (130, 192)]


@pytest.mark.parametrize("fmt", [4, 5, 6, 8, qi.Q8])
@pytest.mark.parametrize("M,K", DQ_SHAPES)
def test_dequant_bit_exact(fmt, M, K):
    say(f"dequant fmt={fmt} M={M} K={K}")
    wl = _workload(fmt, M, K, 1, 11 + M)
    qm = wq.QMat(fmt, wl.codes, wl.scales)
    w = qm.dequant()
    torch.cuda.synchronize()
    got = w.cpu().numpy()
    ref = oracle.dequant_fp8(wl.codes, wl.scales) if fmt == 8 else oracle.dequant_groupwise(qi.code_bits(fmt), wl.codes, wl.scales)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("fmt", [4, 5, 6, qi.Q8])
def test_dequant_every_code_edge_scales(fmt):
    # every code at every position, times +-0, subnormal, largest-normal and ordinary scales
    say(f"dequant edge fmt={fmt}")
    bits = qi.code_bits(fmt)
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    n = hi - lo + 1
    svals = np.array([0.0, -0.0, 2 ** -24, -(2 ** -24), 2 ** -14 - 2 ** -24, 2 ** -14, -1.0, 65504.0,
                      -65504.0, 0.3333, 1e-3, -7.125], dtype=np.float16).view(np.uint16)
    G = svals.size
    M, K = 2 * n + 3, 64 * G
    r = np.arange(M)[:, None]
    k = np.arange(K)[None, :]
    codes = (lo + (r + k) % n).astype(np.int8)
    scales = np.tile(svals, (M, 1))
    scales = np.roll(scales, 1, axis=1) if fmt == 5 else scales
    qm = wq.QMat(fmt, codes, scales)
    got = qm.dequant().cpu().numpy()
    ref = oracle.dequant_groupwise(bits, codes, scales)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_dequant_fp8_every_byte_edge_scales():
    say("dequant fp8 every byte")
    byts = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    rs = np.array([1.0, -0.75, 0.0123, 3.0e-5, 1.7e-38, 1e-40, 2.5e30, 7.0 / 3.0, 0.0, -0.0], np.float32)
    M, K = rs.size, 256
    codes = np.stack([np.roll(np.resize(byts, K), 13 * i) for i in range(M)]).astype(np.uint8)
    qm = wq.QMat(8, codes, rs)
    got = qm.dequant().cpu().numpy()
    ref = oracle.dequant_fp8(codes, rs)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------------ product: tolerance

RUN_SHAPES = [(200, 320), (64, 1024), (1, 64), (130, 192), (257, 2176)]


@pytest.mark.parametrize("route", ["valu", "mfma"])
@pytest.mark.parametrize("fmt", [4, 5, 6, 8, qi.Q8])
@pytest.mark.parametrize("M,K", RUN_SHAPES)
def test_run_parity_small(route, fmt, M, K):
    wl = _workload(fmt, M, K, 16, 100 + M + K + fmt)
    qm = wq.QMat(fmt, wl.codes, wl.scales)
    xd = _x_dev(wl.x)
    for T in (1, 2, 3, 4, 5, 8, 13, 16):
        say(f"run {route} fmt={fmt} M={M} K={K} T={T}")
        y = torch.full((T, M), float("nan"), device="cuda")
        wq.qmat_run_ex(qm.handle, xd[:T], y, T, route=ROUTES[route])
        torch.cuda.synchronize()
        sub = qi.Workload(wl.name, fmt, M, K, T, wl.codes, wl.scales, wl.x[:T])
        _check_y(y, sub, f"{route} fmt={fmt} {M}x{K} T={T}")


@pytest.mark.parametrize("fmt", [4, 5, 6, 8, qi.Q8])
def test_valu_plan_depth(fmt):
    # the vector-ALU route keeps two k units in flight per wave only where both fit in
    # registers: one token per pass, or two for the 4-, 5- and 6-bit formats (the parity test
    # above runs every T through these plans)
    wl = _workload(fmt, 200, 320, 1, 5)
    qm = wq.QMat(fmt, wl.codes, wl.scales)
    two = 1 if fmt in (8, qi.Q8) else 2
    assert [wq.qmat_get_plan(qm.handle, T, wq.QMAT_ROUTE_VALU).depth for T in range(1, 17)] == [2] * two + [1] * (16 - two)
    qm.close()


@pytest.mark.parametrize("fmt", [4, 5, 6, 8, qi.Q8])
@pytest.mark.parametrize("route,T", [("valu", 1), ("valu", 4), ("mfma", 1), ("mfma", 9)])
def test_run_split_shapes_agree(fmt, route, T):
    # every (depth, waves, splits) launch shape gives an in-tolerance result; each is
    # deterministic.  T = 1 on the MFMA route is its single-token specialization.
    M, K = 200, 2176
    wl = _workload(fmt, M, K, T, 7 + fmt + T)
    qm = wq.QMat(fmt, wl.codes, wl.scales)
    xd = _x_dev(wl.x)
    for depth in (1, 2):
        for waves in (1, 2, 4, 8):
            for splits in (1, 2, 3, 5):
                say(f"split {route} fmt={fmt} T={T} depth={depth} waves={waves} splits={splits}")
                y1 = torch.empty((T, M), device="cuda")
                y2 = torch.empty((T, M), device="cuda")
                wq.qmat_run_ex(qm.handle, xd, y1, T, route=ROUTES[route], waves=waves, splits=splits, depth=depth)
                wq.qmat_run_ex(qm.handle, xd, y2, T, route=ROUTES[route], waves=waves, splits=splits, depth=depth)
                torch.cuda.synchronize()
                assert torch.equal(y1, y2)
                _check_y(y1, wl, f"{route} T={T} depth={depth} waves={waves} splits={splits}")


@pytest.mark.parametrize("fmt", [4, 5, 6, 8, qi.Q8])
@pytest.mark.parametrize("route,T", [("valu", 1), ("valu", 3), ("mfma", 1), ("mfma", 6), ("mfma", 16)])
def test_run_tail_plans(fmt, route, T):
    # plans whose trailing tiles are shared by a different number of workgroups than the
    # leading ones (tail_tiles from 1 to all tiles, tail splits 1..8, leading splits 1..3):
    # in tolerance, and deterministic (two calls, same bits)
    M, K = 455, 1472   # 8 tiles, the last one ragged; 12 k units, the last a half unit
    wl = _workload(fmt, M, K, T, 31 + fmt + T)
    qm = wq.QMat(fmt, wl.codes, wl.scales)
    xd = _x_dev(wl.x)
    for depth, waves, splits, tail_tiles, tail_splits in [
            (1, 8, 1, 1, 8), (2, 4, 1, 3, 2), (2, 4, 2, 2, 5), (1, 2, 3, 8, 4), (2, 1, 1, 7, 3),
            (1, 4, 1, 5, 1), (2, 8, 2, 1, 1), (1, 1, 1, 8, 8)]:
        plan = wq.qmat_plan(ROUTES[route], depth, waves, splits, tail_tiles, tail_splits)
        label = f"tail {route} fmt={fmt} T={T} plan={plan.as_tuple()}"
        say(label)
        y1 = torch.full((T, M), float("nan"), device="cuda")
        y2 = torch.full((T, M), float("nan"), device="cuda")
        wq.qmat_run_plan(qm.handle, xd, y1, plan, T=T)
        wq.qmat_run_plan(qm.handle, xd, y2, plan, T=T)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2), label
        _check_y(y1, wl, label)


@pytest.mark.parametrize("case", range(6))
def test_random_shapes_and_plans(case):
    # Seeded random small problems: ragged M, K any multiple of 64 (half units included), every
    # format, T = 1..16, and random valid launch shapes on both small-T routes (waves that get
    # no k unit, trailing splits over all or some tiles, deep splits of short K), each checked
    # against the oracle and for identical bits on a second call.
    rng = np.random.default_rng(1000 + case)
    for i in range(8):
        fmt = int(rng.choice([4, 5, 6, 8, qi.Q8]))
        M = int(rng.integers(1, 700))
        K = 64 * int(rng.integers(1, 40))
        T = int(rng.integers(1, 17))
        route = str(rng.choice(["valu", "mfma"]))
        NT, NU = (M + 63) // 64, (K + 127) // 128
        waves = int(rng.choice([1, 2, 4, 8]))
        depth = int(rng.choice([1, 2]))
        splits = int(rng.integers(1, 9))
        tail_tiles = int(rng.integers(0, NT + 1)) if rng.random() < 0.5 else 0
        tail_splits = int(rng.integers(1, 9))
        # keep within the documented limits: splits * waves <= 64 * NU (and the same for tails)
        while splits * waves > 64 * NU:
            splits = max(1, splits // 2)
        while tail_splits * waves > 64 * NU:
            tail_splits = max(1, tail_splits // 2)
        wl = _workload(fmt, M, K, T, 5000 + 100 * case + i)
        qm = wq.QMat(fmt, wl.codes, wl.scales)
        xd = _x_dev(wl.x)
        plan = wq.qmat_plan(ROUTES[route], depth, waves, splits, tail_tiles, tail_splits)
        label = f"random case={case}.{i} fmt={fmt} M={M} K={K} T={T} plan={plan.as_tuple()}"
        say(label)
        y1 = torch.full((T, M), float("nan"), device="cuda")
        y2 = torch.full((T, M), float("nan"), device="cuda")
        wq.qmat_run_plan(qm.handle, xd, y1, plan, T=T)
        wq.qmat_run_plan(qm.handle, xd, y2, plan, T=T)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2), label
        _check_y(y1, wl, label)
        # and the automatic plan at the same size
        y3 = qm.run(xd)
        torch.cuda.synchronize()
        _check_y(y3, wl, label + " auto")
        qm.close()


@pytest.mark.parametrize("fmt", [4, 5, 6, 8, qi.Q8])
@pytest.mark.parametrize("T", [1, 2, 7, 12, 16])
def test_run_pair_plans(fmt, T):
    # two row tiles per wave (one activation fragment for both): an odd tile count (the last
    # pair has one tile), a ragged last tile and a half k unit; every wave count, both depths,
    # with and without k splits.  In tolerance, deterministic, and the same bits as one tile per
    # wave with the same waves, depth and splits (per tile the arithmetic and the reduction
    # order are the same).
    M, K = 7 * 64 - 9, 1472   # 7 tiles, the last ragged; 12 k units, the last a half unit
    wl = _workload(fmt, M, K, T, 71 + fmt + T)
    qm = wq.QMat(fmt, wl.codes, wl.scales)
    xd = _x_dev(wl.x)
    for depth, waves, splits in [(d, w, 1) for d in (1, 2) for w in (1, 2, 4, 8)] + [
            (1, 4, 3), (2, 8, 2), (1, 1, 5), (2, 2, 8)]:
        pair = wq.qmat_plan(wq.QMAT_ROUTE_MFMA, depth, waves, splits, 0, 1, 2)
        single = wq.qmat_plan(wq.QMAT_ROUTE_MFMA, depth, waves, splits, 0, 1, 1)
        label = f"pair fmt={fmt} T={T} plan={pair.as_tuple()}"
        say(label)
        y1 = torch.full((T, M), float("nan"), device="cuda")
        y2 = torch.full((T, M), float("nan"), device="cuda")
        y0 = torch.full((T, M), float("nan"), device="cuda")
        wq.qmat_run_plan(qm.handle, xd, y1, pair, T=T)
        wq.qmat_run_plan(qm.handle, xd, y2, pair, T=T)
        wq.qmat_run_plan(qm.handle, xd, y0, single, T=T)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2), label
        assert torch.equal(y1, y0), label + " differs from one tile per wave"
        _check_y(y1, wl, label)
    qm.close()


@pytest.mark.parametrize("fmt,T,NT", [(4, 16, 2049), (5, 10, 2049), (6, 12, 2049), (8, 16, 2049), (8, 9, 2049),
                                      (qi.Q8, 13, 2049), (5, 9, 3073), (8, 2, 3073), (qi.Q8, 9, 3073)])
def test_pair_plan_on_head_sized_matrix(fmt, T, NT):
    # the automatic plan of a matrix of >= 2048 row tiles at verify-sized T streams two tiles
    # per wave; with an odd tile count and a ragged last tile it matches the oracle on sampled
    # rows (the last tile included) and one tile per wave bit for bit
    M, K = NT * 64 - 7, 320
    wl = _workload(fmt, M, K, T, 91 + fmt)
    qm = wq.QMat(fmt, wl.codes, wl.scales)
    p = wq.qmat_get_plan(qm.handle, T)
    say(f"head-sized fmt={fmt} T={T} auto plan {p.as_tuple()}")
    assert p.route == wq.QMAT_ROUTE_MFMA and p.tiles == 2 and p.splits == 1 and p.tail_tiles == 0
    # two tiles per wave from each format's crossover, one below: with >= 3072 tiles FP8 2, Q8
    # and Q5 9, Q4 and Q6 10; with fewer the 8-bit formats 9, the others 10
    first = {8: 2, qi.Q8: 9, 5: 9}.get(fmt, 10) if NT >= 3072 else (9 if fmt in (8, qi.Q8) else 10)
    assert [wq.qmat_get_plan(qm.handle, t).tiles for t in range(1, 17)] == [1] * (first - 1) + [2] * (17 - first)
    xd = _x_dev(wl.x)
    y = torch.full((T, M), float("nan"), device="cuda")
    y0 = torch.full((T, M), float("nan"), device="cuda")
    wq.qmat_run(qm.handle, xd, y, T=T)
    wq.qmat_run_plan(qm.handle, xd, y0, wq.qmat_plan(p.route, p.depth, p.waves, 1, 0, 1, 1), T=T)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any()
    assert torch.equal(y, y0)
    rows = sorted(set(_sample_rows(M, n=400, seed=3)) | set(range(M - 57, M)))
    _check_y(y, wl, f"head-sized fmt={fmt} T={T}", rows=rows)
    qm.close()


def test_trailing_split_plan_on_gate_up_rows():
    # 544 row tiles on 256 compute units: the 32 trailing tiles are split along K, 8 ways at
    # T = 1 and 4 ways from T = 2; the result matches the oracle on sampled and trailing rows
    M, K = 34816 - 5, 1024
    wl = _workload(4, M, K, 8, 93)
    qm = wq.QMat(4, wl.codes, wl.scales)
    for T, st in ((1, 8), (4, 4), (8, 4), (12, 4)):
        p = wq.qmat_get_plan(qm.handle, T)
        say(f"gate+up rows T={T} auto plan {p.as_tuple()}")
        assert (p.tail_tiles, p.tail_splits) == (32, st)
    for T in (1, 8):
        xd = _x_dev(wl.x[:T])
        y = torch.full((T, M), float("nan"), device="cuda")
        wq.qmat_run(qm.handle, xd, y, T=T)
        torch.cuda.synchronize()
        assert not torch.isnan(y).any()
        sub = qi.Workload(wl.name, 4, M, K, T, wl.codes, wl.scales, wl.x[:T])
        _check_y(y, sub, f"gate+up rows T={T}", rows=sorted(set(_sample_rows(M, n=300, seed=4)) | set(range(M - 2100, M))))
    qm.close()


@pytest.mark.parametrize("fmt,K,T", [(5, 2176, 1), (5, 2176, 4), (4, 2176, 8), (8, 1152, 2)])
def test_short_k_plan_one_unit_slices(fmt, K, T):
    # a few hundred row tiles of very short K: the automatic plan splits every tile until each
    # wave holds one k unit at most (some waves empty), and matches the oracle on every row and
    # a plan with fewer, fuller slices to rounding
    M = 5120 - 9
    wl = _workload(fmt, M, K, T, 47 + K)
    qm = wq.QMat(fmt, wl.codes, wl.scales)
    NU = K // 128
    p = wq.qmat_get_plan(qm.handle, T)
    say(f"short K fmt={fmt} K={K} T={T} auto plan {p.as_tuple()}")
    assert p.route == wq.QMAT_ROUTE_MFMA and p.tail_tiles == 0 and p.splits > 1
    assert -(-NU // (p.splits * p.waves)) == 1 and p.splits * p.waves >= NU
    xd = _x_dev(wl.x)
    y = torch.full((T, M), float("nan"), device="cuda")
    y1 = torch.full((T, M), float("nan"), device="cuda")
    wq.qmat_run(qm.handle, xd, y, T=T)
    wq.qmat_run_plan(qm.handle, xd, y1, wq.qmat_plan(p.route, 1, 4, 1, 0, 1, 1), T=T)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any()
    _check_y(y, wl, f"short K fmt={fmt} K={K} T={T}")
    torch.testing.assert_close(y, y1, rtol=1e-5, atol=1e-5)
    qm.close()


def test_run_plan_rejects_bad_fields():
    say("run_plan errors")
    wl = _workload(4, 130, 256, 1, 5)
    qm = wq.QMat(4, wl.codes, wl.scales)
    xd = _x_dev(wl.x)
    y = torch.empty((1, 130), device="cuda")
    NT = 3
    bad = [(0, 1, 4, 1, 0, 1), (2, 3, 4, 1, 0, 1), (2, 1, 3, 1, 0, 1), (2, 1, 4, 0, 0, 1),
           (2, 1, 4, 1, NT + 1, 1), (2, 1, 4, 1, -1, 1), (2, 1, 4, 1, 1, 0)]
    for fields in bad:
        with pytest.raises(wq.QmatError) as e:
            wq.qmat_run_plan(qm.handle, xd, y, wq.qmat_plan(*fields), T=1)
        assert e.value.status == wq.QMAT_EINVAL, fields
    # tiles: 1 or 2; two tiles per wave only on the MFMA route without a trailing split
    for fields in [(2, 1, 4, 1, 0, 1, 3), (2, 1, 4, 1, 0, 1, -1), (1, 1, 4, 1, 0, 1, 2), (2, 1, 4, 1, 1, 2, 2)]:
        with pytest.raises(wq.QmatError) as e:
            wq.qmat_run_plan(qm.handle, xd, y, wq.qmat_plan(*fields), T=1)
        assert e.value.status == wq.QMAT_EINVAL, fields
    with pytest.raises(wq.QmatError) as e:  # more splits than the workspace holds
        wq.qmat_run_plan(qm.handle, xd, y, wq.qmat_plan(2, 1, 1, 1, 2, 64 * 2), T=16)
    assert e.value.status == wq.QMAT_ESIZE


@pytest.mark.parametrize("fmt", [4, 6, 8, qi.Q8])
def test_row_views(fmt):
    # views over tile-aligned row ranges of one packed matrix (gate / up halves, a ragged last
    # range, a single partial tile) give the sub-matrix's product and dequantization; the view
    # outlives its parent handle
    M, K, T = 455, 704, 5
    wl = _workload(fmt, M, K, 40, 41 + fmt)
    qm = wq.QMat(fmt, wl.codes, wl.scales)
    xd = _x_dev(wl.x)
    for row0, rows in [(0, 192), (192, 263), (128, 64), (448, 7), (64, 1), (0, M)]:
        say(f"view fmt={fmt} rows [{row0}, {row0 + rows})")
        v = wq.qmat_create_view(qm.handle, row0, rows)
        sub = qi.Workload("v", fmt, rows, K, T, wl.codes[row0:row0 + rows], wl.scales[row0:row0 + rows], wl.x)
        for Tr in (1, T, 40):  # 40: the prefill GEMM route on the view
            y = torch.full((Tr, rows), float("nan"), device="cuda")
            wq.qmat_run(v, xd[:Tr], y, T=Tr)
            torch.cuda.synchronize()
            _check_y(y, qi.Workload("v", fmt, rows, K, Tr, sub.codes, sub.scales, wl.x[:Tr]), f"view {row0}+{rows} T={Tr}")
        w = torch.empty((rows, K), device="cuda")
        wq.qmat_dequant(v, w)
        torch.cuda.synchronize()
        ref = oracle.dequant_fp8(sub.codes, sub.scales) if fmt == 8 else \
            oracle.dequant_groupwise(qi.code_bits(fmt), sub.codes, sub.scales)
        assert np.array_equal(w.cpu().numpy().view(np.uint32), ref.view(np.uint32))
        wq.qmat_destroy(v)
    v = wq.qmat_create_view(qm.handle, 256, 199)
    qm.close()  # the parent handle goes first; the packed blob (qm.packed) stays alive
    y = torch.empty((T, 199), device="cuda")
    wq.qmat_run(v, xd[:T], y, T=T)
    torch.cuda.synchronize()
    _check_y(y, qi.Workload("v", fmt, 199, K, T, wl.codes[256:], wl.scales[256:], wl.x[:T]), "view after parent")
    wq.qmat_destroy(v)
    parent = wq.qmat_create(fmt, M, K, qm.packed)
    for row0, rows in [(1, 64), (-64, 64), (0, 0), (448, 8), (512, 1)]:
        with pytest.raises(wq.QmatError) as e:
            wq.qmat_create_view(parent, row0, rows)
        assert e.value.status == wq.QMAT_ESHAPE, (row0, rows)
    wq.qmat_destroy(parent)


# ------------------------------------------------------------------ prefill GEMM route

GEMM_SHAPES = [(200, 320), (64, 1024), (1, 64), (257, 2176), (300, 192)]


@pytest.mark.parametrize("fmt", [4, 5, 6, 8, qi.Q8])
@pytest.mark.parametrize("M,K", GEMM_SHAPES)
def test_gemm_parity(fmt, M, K):
    # token counts below, at and across the 64-token tile (ragged last tile), on the explicit
    # GEMM route and (T > 16) the automatic one
    Tmax = 130
    wl = _workload(fmt, M, K, Tmax, 500 + M + K + fmt)
    qm = wq.QMat(fmt, wl.codes, wl.scales)
    xd = _x_dev(wl.x)
    for T in (1, 17, 64, 100, 130):
        say(f"gemm fmt={fmt} M={M} K={K} T={T}")
        y = torch.full((T, M), float("nan"), device="cuda")
        if T > 16 and T % 2:
            wq.qmat_run(qm.handle, xd[:T], y, T=T)
        else:
            wq.qmat_run_ex(qm.handle, xd[:T], y, T, route=wq.QMAT_ROUTE_GEMM)
        torch.cuda.synchronize()
        sub = qi.Workload(wl.name, fmt, M, K, T, wl.codes, wl.scales, wl.x[:T])
        _check_y(y, sub, f"gemm fmt={fmt} {M}x{K} T={T}")


@pytest.mark.parametrize("fmt", [4, 5, 6, 8, qi.Q8])
def test_gemm_bit_exact_on_exact_inputs(fmt):
    M, K, T = 130, 1024, 70
    say(f"gemm exact fmt={fmt}")
    wl = _exact_workload(fmt, M, K, T, 9)
    qm = wq.QMat(fmt, wl.codes, wl.scales)
    y = torch.empty((T, M), device="cuda")
    wq.qmat_run(qm.handle, _x_dev(wl.x), y, T=T)
    torch.cuda.synchronize()
    y_ref, _ = oracle.gemv(fmt, wl.codes, wl.scales, wl.x)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y_ref)


def test_gemm_plan_and_graph_replay():
    import gc
    gc.collect()
    wl = _workload(4, 320, 640, 96, 3)
    qm = wq.QMat(4, wl.codes, wl.scales)
    assert wq.qmat_get_plan(qm.handle, 96).route == wq.QMAT_ROUTE_GEMM
    assert wq.qmat_get_plan(qm.handle, 16).route == wq.QMAT_ROUTE_MFMA
    xd = _x_dev(wl.x)
    y_eager = torch.empty((96, 320), device="cuda")
    wq.qmat_run(qm.handle, xd, y_eager, T=96)
    y = torch.empty_like(y_eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wq.qmat_run(qm.handle, xd, y, T=96)
    for i in range(3):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), i
        wq.qmat_run(qm.handle, xd, y_eager, T=96)  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("fmt", [4, 5, 6, 8, qi.Q8])
def test_gemm_split_k(fmt):
    # k splits forced through explicit plans (ragged unit counts per split, ragged last token
    # tile): each within tolerance, each repeatable bit for bit (fixed summation order, counters
    # reset by the last wave), and an automatic split on a narrow matrix
    M, K, Tmax = 200, 2048, 130
    wl = _workload(fmt, M, K, Tmax, 77 + fmt)
    qm = wq.QMat(fmt, wl.codes, wl.scales)
    xd = _x_dev(wl.x)
    for T in (17, 64, 130):
        sub = qi.Workload(wl.name, fmt, M, K, T, wl.codes, wl.scales, wl.x[:T])
        for S in (2, 3, 5, 16):
            say(f"gemm split fmt={fmt} T={T} S={S}")
            plan = wq.qmat_plan(wq.QMAT_ROUTE_GEMM, 1, 4, S, 0, 1)
            y1 = torch.full((T, M), float("nan"), device="cuda")
            y2 = torch.full((T, M), float("nan"), device="cuda")
            wq.qmat_run_plan(qm.handle, xd[:T], y1, plan, T=T)
            wq.qmat_run_plan(qm.handle, xd[:T], y2, plan, T=T)
            torch.cuda.synchronize()
            assert torch.equal(y1, y2), (T, S)
            _check_y(y1, sub, f"gemm split fmt={fmt} T={T} S={S}")
    p = wq.qmat_get_plan(qm.handle, 64)
    assert p.route == wq.QMAT_ROUTE_GEMM and p.splits > 1, p.as_tuple()
    y = torch.full((64, M), float("nan"), device="cuda")
    wq.qmat_run(qm.handle, xd[:64], y, T=64)
    torch.cuda.synchronize()
    _check_y(y, qi.Workload(wl.name, fmt, M, K, 64, wl.codes, wl.scales, wl.x[:64]), f"gemm auto split fmt={fmt}")
    qm.close()


@pytest.mark.parametrize("fmt", [4, 8])
def test_gemm_block_order_ragged_patches(fmt):
    # more than one 8 x 8 patch of (row block, token tile) work in both directions, each with a
    # ragged remainder: 10 row blocks (37 tiles, the last partial) x 10 token tiles (T = 581)
    M, K, T = 64 * 37 - 20, 256, 581
    say(f"gemm patches fmt={fmt}")
    wl = _workload(fmt, M, K, T, 123 + fmt)
    qm = wq.QMat(fmt, wl.codes, wl.scales)
    y = torch.full((T, M), float("nan"), device="cuda")
    wq.qmat_run(qm.handle, _x_dev(wl.x), y, T=T)
    torch.cuda.synchronize()
    assert wq.qmat_get_plan(qm.handle, T).splits == 1
    _check_y(y, wl, f"gemm patches fmt={fmt}")
    qm.close()


@pytest.mark.parametrize("fmt", [4, 8])
def test_gemm_split_k_bit_exact_and_graph_replay(fmt):
    M, K, T = 130, 2048, 70
    wl = _exact_workload(fmt, M, K, T, 19)
    qm = wq.QMat(fmt, wl.codes, wl.scales)
    xd = _x_dev(wl.x)
    y_ref, _ = oracle.gemv(fmt, wl.codes, wl.scales, wl.x)
    plan = wq.qmat_plan(wq.QMAT_ROUTE_GEMM, 1, 4, 3, 0, 1)
    y = torch.empty((T, M), device="cuda")
    wq.qmat_run_plan(qm.handle, xd, y, plan, T=T)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y_ref)
    yg = torch.empty_like(y)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wq.qmat_run_plan(qm.handle, xd, yg, plan, T=T)
    for i in range(3):
        yg.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, y), i
        wq.qmat_run_plan(qm.handle, xd, y, plan, T=T)  # eager work between replays
        torch.cuda.synchronize()
    del g
    qm.close()


def test_gemm_split_k_argument_errors():
    wl = _workload(4, 200, 512, 20, 5)
    qm = wq.QMat(4, wl.codes, wl.scales)
    xd = _x_dev(wl.x)
    y = torch.empty((20, 200), device="cuda")
    for S, status in [(0, wq.QMAT_EINVAL), (5, wq.QMAT_EINVAL), (17, wq.QMAT_EINVAL)]:  # NU = 4
        with pytest.raises(wq.QmatError) as e:
            wq.qmat_run_plan(qm.handle, xd, y, wq.qmat_plan(wq.QMAT_ROUTE_GEMM, 1, 4, S, 0, 1), T=20)
        assert e.value.status == status, S
    big = 4 << 20  # 16 Mi floats of workspace would be needed: rejected on the host, nothing launched
    T = big // (4 * 256) + 64
    xb = torch.zeros((T, 512), dtype=torch.bfloat16, device="cuda")
    yb = torch.empty((T, 200), device="cuda")
    with pytest.raises(wq.QmatError) as e:
        wq.qmat_run_plan(qm.handle, xb, yb, wq.qmat_plan(wq.QMAT_ROUTE_GEMM, 1, 4, 4, 0, 1), T=T)
    assert e.value.status == wq.QMAT_ESIZE
    qm.close()


def _exact_workload(fmt, M, K, T, seed):
    """Inputs whose products and partial sums are all exact in fp32: small integer bf16
    activations and power-of-two scales (FP8: integer-valued E4M3 bytes)."""
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.integers(-4, 5, (T, K)).astype(np.float32)).to(torch.bfloat16)
    x_bits = x.view(torch.int16).numpy().view(np.uint16)
    if fmt == 8:
        ints = rng.integers(-16, 17, (M, K)).astype(np.float32)
        codes = torch.from_numpy(ints).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        scales = (2.0 ** rng.integers(-6, 3, M)).astype(np.float32)
    else:
        bits = qi.code_bits(fmt)
        lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
        codes = rng.integers(lo, hi + 1, (M, K)).astype(np.int8)
        sg = np.where(rng.random((M, K // 64)) < 0.5, -1.0, 1.0)
        scales = (sg * 2.0 ** rng.integers(-2, 2, (M, K // 64))).astype(np.float16).view(np.uint16)
    return qi.Workload("exact", fmt, M, K, T, codes, scales, x_bits)


@pytest.mark.parametrize("route", ["valu", "mfma"])
@pytest.mark.parametrize("fmt", [4, 5, 6, 8, qi.Q8])
def test_run_bit_exact_on_exact_inputs(route, fmt):
    M, K = 130, 1024
    for T in (1, 4, 8, 16):
        say(f"exact {route} fmt={fmt} T={T}")
        wl = _exact_workload(fmt, M, K, T, 3 + T)
        qm = wq.QMat(fmt, wl.codes, wl.scales)
        y = torch.empty((T, M), device="cuda")
        wq.qmat_run_ex(qm.handle, _x_dev(wl.x), y, T, route=ROUTES[route])
        torch.cuda.synchronize()
        y_ref, _ = oracle.gemv(fmt, wl.codes, wl.scales, wl.x)
        assert np.array_equal(y.cpu().numpy().astype(np.float64), y_ref)


# ------------------------------------------------------------------ degenerate inputs

@pytest.mark.parametrize("fmt", [4, 5, 6, 8, qi.Q8])
def test_zero_and_sparse_codes(fmt):
    # all-zero codes give exactly zero; one nonzero code per row gives that single product
    M, K, T = 70, 640, 8
    wl = _workload(fmt, M, K, T, 21)
    codes = np.zeros_like(wl.codes)
    rng = np.random.default_rng(5)
    cols = rng.integers(0, K, M)
    for i in range(1, M):
        b = qi.code_bits(fmt)
        codes[i, cols[i]] = (0x38 if fmt == 8 else (-(1 << (b - 1)) if i % 2 else (1 << (b - 1)) - 1))
    for route in ("valu", "mfma"):
        say(f"sparse {route} fmt={fmt}")
        qm = wq.QMat(fmt, codes, wl.scales)
        y = torch.empty((T, M), device="cuda")
        wq.qmat_run_ex(qm.handle, _x_dev(wl.x), y, T, route=ROUTES[route])
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        assert np.all(got[:, 0] == 0)
        _check_y(y, qi.Workload("s", fmt, M, K, T, codes, wl.scales, wl.x), f"sparse {route}")


@pytest.mark.parametrize("T", [1, 4, 8, 12])
def test_q4_offset_operands_on_zero_and_sparse_rows(T):
    # QMAT_ROUTE_MFMA_OFFSET: Q4 reaches the matrix cores as offset-binary operands
    # (code + 8) / 512 up to 8 tokens, the offset taken out per group by subtracting the same
    # MFMA sum over a constant operand.  Rows of zero codes must still give exactly 0, and rows
    # that are 90-99% zero codes stay within the tolerance next to activations with outlier
    # channels of 256x on 1% of K (not adversarial: the outliers fall on codes of any value)
    M, K = 96, 2048
    wl = _workload(4, M, K, T, 77 + T)
    rng = np.random.default_rng(9 + T)
    codes = wl.codes.copy()
    codes[:16] = 0
    for i in range(16, M):
        keep = 0.10 if i < 56 else 0.01
        codes[i, rng.random(K) >= keep] = 0
    x = torch.from_numpy(wl.x.view(np.int16).copy()).view(torch.bfloat16).float()
    outl = rng.choice(K, K // 100, replace=False)
    x[:, outl] *= 256.0
    xb = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    scales = wl.scales.copy()
    scales[:16] = np.float16(1000.0).view(np.uint16)
    qm = wq.QMat(4, codes, scales)
    y = torch.full((T, M), float("nan"), device="cuda")
    wq.qmat_run_ex(qm.handle, _x_dev(xb), y, T, route=wq.QMAT_ROUTE_MFMA_OFFSET)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    assert np.all(got[:, :16] == 0)
    worst = _check_y(y, qi.Workload("q4s", 4, M, K, T, codes, scales, xb), f"q4 sparse rows T={T}")
    say(f"q4 sparse rows T={T}: worst ratio {worst:.3g}")
    qm.close()


def test_default_route_keeps_the_bound_on_adversarial_q4_rows():
    # rows with half their codes zero, activations of 2^12 exactly on those zero codes and 2^-6
    # elsewhere: sum|w x| only sees the small products.  The automatic route (two's complement
    # operands) keeps the bound at T = 1-8, one and two tiles per wave; the offset-operand
    # route's sums see the large activations, and its ratio to the bound is reported only.
    M, K = 128, 1024
    rng = np.random.default_rng(123)
    codes = rng.integers(1, 8, (M, K)).astype(np.int8) * np.where(rng.random((M, K)) < 0.5, -1, 1).astype(np.int8)
    zero = rng.random(K) < 0.5
    codes[:, zero] = 0
    scales = np.full((M, K // 64), np.float16(0.5)).view(np.uint16)
    qm = wq.QMat(4, codes, scales)
    for T in (1, 4, 8):
        x = np.where(zero, 2.0 ** 12, 2.0 ** -6).astype(np.float32)[None, :].repeat(T, 0)
        x *= np.where(rng.random((T, K)) < 0.5, -1.0, 1.0)
        xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        wl = qi.Workload("adv", 4, M, K, T, codes, scales, xb)
        ya = torch.full((T, M), float("nan"), device="cuda")
        yp = torch.full((T, M), float("nan"), device="cuda")
        yo = torch.full((T, M), float("nan"), device="cuda")
        wq.qmat_run(qm.handle, _x_dev(xb), ya, T=T)
        wq.qmat_run_plan(qm.handle, _x_dev(xb), yp, wq.qmat_plan(wq.QMAT_ROUTE_MFMA, 1, 2, 1, 0, 1, 2), T=T)
        wq.qmat_run_ex(qm.handle, _x_dev(xb), yo, T, route=wq.QMAT_ROUTE_MFMA_OFFSET)
        torch.cuda.synchronize()
        worst = _check_y(ya, wl, f"automatic route T={T}")
        _check_y(yp, wl, f"automatic route pair plan T={T}")
        y_ref, A = oracle.gemv(4, codes, scales, xb)
        _, off_worst, _ = oracle.check(yo.cpu().numpy().astype(np.float64), y_ref, A)
        say(f"adversarial Q4 T={T}: automatic route worst ratio {worst:.3g}, offset-operand route {off_worst:.3g}")
    qm.close()


@pytest.mark.parametrize("fmt", [5, 6, 8, qi.Q8])
@pytest.mark.parametrize("T", [1, 8, 16])
def test_automatic_route_keeps_the_bound_next_to_large_activations_on_zero_codes(fmt, T):
    # the same adversarial input for every other format: zero codes (FP8: +0 and -0 bytes)
    # under activations of 2^12, small products elsewhere; a zero code contributes an exact 0
    # on the signed operands, so the bound holds however large its activation
    M, K = 96, 1024
    rng = np.random.default_rng(200 + fmt + T)
    zero = rng.random(K) < 0.5
    if fmt == 8:
        mag = rng.integers(0x20, 0x58, (M, K)).astype(np.uint8)
        codes = mag | np.where(rng.random((M, K)) < 0.5, 0x80, 0x00).astype(np.uint8)
        codes[:, zero] = np.where(rng.random((M, int(zero.sum()))) < 0.5, 0x00, 0x80).astype(np.uint8)
        scales = np.full(M, 0.25, np.float32)
    else:
        qmax = (1 << (qi.code_bits(fmt) - 1)) - 1
        codes = rng.integers(1, qmax + 1, (M, K)).astype(np.int8) * np.where(rng.random((M, K)) < 0.5, -1, 1).astype(np.int8)
        codes[:, zero] = 0
        scales = np.full((M, K // 64), np.float16(0.5)).view(np.uint16)
    x = np.where(zero, 2.0 ** 12, 2.0 ** -6).astype(np.float32)[None, :].repeat(T, 0)
    x *= np.where(rng.random((T, K)) < 0.5, -1.0, 1.0)
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    qm = wq.QMat(fmt, codes, scales)
    y = torch.full((T, M), float("nan"), device="cuda")
    wq.qmat_run(qm.handle, _x_dev(xb), y, T=T)
    torch.cuda.synchronize()
    worst = _check_y(y, qi.Workload("adv", fmt, M, K, T, codes, scales, xb), f"adversarial fmt={fmt} T={T}")
    say(f"adversarial fmt={fmt} T={T}: worst ratio {worst:.3g}")
    qm.close()


@pytest.mark.parametrize("fmt", [4, 5, 8])
def test_offset_route_parity_and_shared_kernels(fmt):
    # QMAT_ROUTE_MFMA_OFFSET: in tolerance on random inputs, one tile per wave and two (the
    # same bits), and bit-exact on exact-arithmetic inputs at every T; for every format but Q4,
    # and for Q4 above 8 tokens, it runs the automatic route's kernels (the same bits)
    M, K = 200, 1536
    for T in (1, 3, 6, 8, 12):
        wl = _workload(fmt, M, K, T, 300 + T)
        qm = wq.QMat(fmt, wl.codes, wl.scales)
        yo = torch.full((T, M), float("nan"), device="cuda")
        ya = torch.full((T, M), float("nan"), device="cuda")
        y1 = torch.full((T, M), float("nan"), device="cuda")
        y2 = torch.full((T, M), float("nan"), device="cuda")
        wq.qmat_run_ex(qm.handle, _x_dev(wl.x), yo, T, route=wq.QMAT_ROUTE_MFMA_OFFSET)
        wq.qmat_run(qm.handle, _x_dev(wl.x), ya, T=T)
        p = wq.qmat_get_plan(qm.handle, T, wq.QMAT_ROUTE_MFMA_OFFSET)
        assert p.route == wq.QMAT_ROUTE_MFMA_OFFSET
        wq.qmat_run_plan(qm.handle, _x_dev(wl.x), y1, wq.qmat_plan(wq.QMAT_ROUTE_MFMA_OFFSET, 1, 2, 1, 0, 1, 1), T=T)
        wq.qmat_run_plan(qm.handle, _x_dev(wl.x), y2, wq.qmat_plan(wq.QMAT_ROUTE_MFMA_OFFSET, 1, 2, 1, 0, 1, 2), T=T)
        torch.cuda.synchronize()
        _check_y(yo, wl, f"offset fmt={fmt} T={T}")
        assert torch.equal(y1, y2)
        if fmt != 4 or T > 8:
            assert torch.equal(yo, ya)
        qm.close()
        ex = _exact_workload(fmt, 130, 1024, T, 7 + T)
        qe = wq.QMat(fmt, ex.codes, ex.scales)
        ye = torch.empty((T, 130), device="cuda")
        wq.qmat_run_ex(qe.handle, _x_dev(ex.x), ye, T, route=wq.QMAT_ROUTE_MFMA_OFFSET)
        torch.cuda.synchronize()
        y_ref, _ = oracle.gemv(fmt, ex.codes, ex.scales, ex.x)
        assert np.array_equal(ye.cpu().numpy().astype(np.float64), y_ref)
        qe.close()


# FP8 row scales the API accepts (any finite fp32) that the seeded workloads never produce:
# negative, +0, -0, subnormal, the smallest normal and large magnitudes
FP8_EDGE_ROW_SCALES = np.array([-0.0123, 0.0, -0.0, 1.0e-40, -3.0e-42, 2.0 ** -126, -1.0e30, 7.5e29,
                                -1.0, 1.0, 2.0 ** -149, -(2.0 ** -149)], dtype=np.float32)


@pytest.mark.parametrize("route", ["valu", "mfma"])
def test_fp8_edge_row_scales_product(route):
    M, K = 200, 640
    for T in (1, 8, 16):
        wl = _workload(8, M, K, T, 40 + T)
        scales = wl.scales.copy()
        scales[: len(FP8_EDGE_ROW_SCALES)] = FP8_EDGE_ROW_SCALES
        scales[64: 64 + len(FP8_EDGE_ROW_SCALES)] = FP8_EDGE_ROW_SCALES[::-1]
        scales[-len(FP8_EDGE_ROW_SCALES):] = FP8_EDGE_ROW_SCALES
        say(f"fp8 edge row scales {route} T={T}")
        qm = wq.QMat(8, wl.codes, scales)
        y = torch.full((T, M), float("nan"), device="cuda")
        wq.qmat_run_ex(qm.handle, _x_dev(wl.x), y, T, route=ROUTES[route])
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        assert np.all(got[:, 1] == 0) and np.all(got[:, 2] == 0)  # zero row scales give zero
        _check_y(y, qi.Workload("e", 8, M, K, T, wl.codes, scales, wl.x), f"fp8 edge scales {route} T={T}")
        qm.close()


# FP16 group scales: +-0, the smallest subnormal, the largest subnormal, the smallest normal,
# +-65504 and ordinary negative values, spread over every group position of some rows
HALF_EDGE_SCALES = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x83FF, 0x0400, 0x8400, 0x7BFF,
                             0xFBFF, 0xBC00, 0x3C00, 0xA266], dtype=np.uint16)


@pytest.mark.parametrize("route", ["valu", "mfma"])
@pytest.mark.parametrize("fmt", [4, 5, 6, qi.Q8])
def test_groupwise_edge_scales_product(route, fmt):
    M, K = 150, 1536
    G = K // 64
    for T in (1, 8):
        wl = _workload(fmt, M, K, T, 60 + fmt + T)
        scales = wl.scales.copy()
        n = len(HALF_EDGE_SCALES)
        for i in range(0, M, 3):
            scales[i] = HALF_EDGE_SCALES[(np.arange(G) + i) % n]
        say(f"groupwise edge scales {route} fmt={fmt} T={T}")
        qm = wq.QMat(fmt, wl.codes, scales)
        y = torch.full((T, M), float("nan"), device="cuda")
        wq.qmat_run_ex(qm.handle, _x_dev(wl.x), y, T, route=ROUTES[route])
        torch.cuda.synchronize()
        _check_y(y, qi.Workload("e", fmt, M, K, T, wl.codes, scales, wl.x), f"edge scales {route} fmt={fmt} T={T}")
        qm.close()


@pytest.mark.parametrize("fmt,T", [(4, 16), (8, 1), (qi.Q8, 5), (6, 3)])
def test_largest_k(fmt, T):
    # K at the largest size the library accepts (2^20: 8192 k units per tile) with a ragged row
    # count, on the automatic plan (k splits of a narrow matrix) and an explicit deep split with
    # a trailing-tile split; every output element against the oracle
    M, K = 70, 1 << 20
    wl = _workload(fmt, M, K, T, 910 + fmt + T)
    qm = wq.QMat(fmt, wl.codes, wl.scales)
    xd = _x_dev(wl.x)
    say(f"largest K fmt={fmt} T={T} auto plan {wq.qmat_get_plan(qm.handle, T).as_tuple()}")
    y = qm.run(xd)
    torch.cuda.synchronize()
    _check_y(y, wl, f"K=2^20 fmt={fmt} T={T} auto")
    plan = wq.qmat_plan(wq.QMAT_ROUTE_MFMA, 2, 8, 8, 1, 5)
    say(f"largest K fmt={fmt} T={T} plan {plan.as_tuple()}")
    y2 = torch.full((T, M), float("nan"), device="cuda")
    wq.qmat_run_plan(qm.handle, xd, y2, plan, T=T)
    torch.cuda.synchronize()
    _check_y(y2, wl, f"K=2^20 fmt={fmt} T={T} plan")
    qm.close()


def test_largest_k_gemm():
    # the prefill GEMM route at the largest K (its activation staging offsets and k splits over
    # 8192 units), T = 80 (a ragged second token tile), every output against the oracle
    M, K, T = 70, 1 << 20, 80
    wl = _workload(4, M, K, T, 977)
    qm = wq.QMat(4, wl.codes, wl.scales)
    xd = _x_dev(wl.x)
    for S in (0, 16):
        say(f"largest K GEMM T={T} splits={S}")
        y = torch.full((T, M), float("nan"), device="cuda")
        wq.qmat_run_ex(qm.handle, xd, y, T, route=wq.QMAT_ROUTE_GEMM, splits=S)
        torch.cuda.synchronize()
        _check_y(y, wl, f"K=2^20 GEMM splits={S}")
    qm.close()


def test_t_zero_is_noop_and_bad_args():
    wl = _workload(4, 64, 128, 1, 1)
    qm = wq.QMat(4, wl.codes, wl.scales)
    xd = _x_dev(wl.x)
    y = torch.full((1, 64), 7.0, device="cuda")
    wq.qmat_run(qm.handle, xd, y, T=0)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    with pytest.raises(wq.QmatError) as e:  # beyond the largest GEMM launch: rejected on the host
        wq.qmat_run(qm.handle, xd, y, T=65535 * 64 + 1)
    assert e.value.status == wq.QMAT_ESHAPE
    with pytest.raises(wq.QmatError) as e:  # the small-T routes stop at 16
        wq.qmat_run_ex(qm.handle, xd, y, 17, route=wq.QMAT_ROUTE_MFMA)
    assert e.value.status == wq.QMAT_ESHAPE
    with pytest.raises(wq.QmatError) as e:
        wq.qmat_run(qm.handle, xd, y, T=-1)
    assert e.value.status == wq.QMAT_ESHAPE
    xbig = torch.zeros(200, dtype=torch.bfloat16, device="cuda")
    assert wq.lib().qmat_run(qm.handle, xbig.data_ptr() + 2, y.data_ptr(), 1, None) == wq.QMAT_EINVAL
    with pytest.raises(wq.QmatError) as e:
        wq.qmat_run_ex(qm.handle, xd, y, 1, route=5)
    assert e.value.status == wq.QMAT_EINVAL
    with pytest.raises(wq.QmatError) as e:
        wq.qmat_run_ex(qm.handle, xd, y, 1, waves=3)
    assert e.value.status == wq.QMAT_EINVAL


def test_create_rejects_wrong_size():
    wl = _workload(6, 64, 128, 1, 1)
    blob = torch.from_numpy(wq.qmat_pack(6, wl.codes, wl.scales)).cuda()
    with pytest.raises(wq.QmatError) as e:
        wq.qmat_create(6, 64, 192, blob)
    assert e.value.status == wq.QMAT_ESIZE


def test_graph_replay_matches_eager():
    # the split-K path resets its own arrival counters, so graph replays need no memset.
    # Garbage from earlier tests is collected first: a handle freed (hipFree) while the
    # stream captures would invalidate the capture.
    import gc
    gc.collect()
    M, K, T = 320, 4352, 4
    wl = _workload(5, M, K, T, 77)
    qm = wq.QMat(5, wl.codes, wl.scales)
    xd = _x_dev(wl.x)
    y_eager = torch.empty((T, M), device="cuda")
    wq.qmat_run_ex(qm.handle, xd, y_eager, T, waves=4, splits=5)
    torch.cuda.synchronize()
    y = torch.empty((T, M), device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        wq.qmat_run_ex(qm.handle, xd, y, T, waves=4, splits=5, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wq.qmat_run_ex(qm.handle, xd, y, T, waves=4, splits=5)
    for i in range(4):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {i}"
        wq.qmat_run_ex(qm.handle, xd, y_eager, T, waves=4, splits=5)  # eager work between replays
        torch.cuda.synchronize()


def test_pair_plan_graph_replay_matches_eager():
    # two tiles per wave with k splits: both tiles of a pair count in on their own arrival
    # counters and reset them, so replays need no memset
    import gc
    gc.collect()
    M, K, T = 7 * 64 - 9, 4352, 16
    wl = _workload(6, M, K, T, 78)
    qm = wq.QMat(6, wl.codes, wl.scales)
    xd = _x_dev(wl.x)
    plan = wq.qmat_plan(wq.QMAT_ROUTE_MFMA, 1, 4, 3, 0, 1, 2)
    y_eager = torch.empty((T, M), device="cuda")
    wq.qmat_run_plan(qm.handle, xd, y_eager, plan, T=T)
    torch.cuda.synchronize()
    _check_y(y_eager, wl, "pair graph eager")
    y = torch.empty((T, M), device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        wq.qmat_run_plan(qm.handle, xd, y, plan, T=T, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wq.qmat_run_plan(qm.handle, xd, y, plan, T=T, stream=torch.cuda.current_stream())
    for i in range(4):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {i}"
        wq.qmat_run_plan(qm.handle, xd, y_eager, plan, T=T)  # eager work between replays
        torch.cuda.synchronize()


# ------------------------------------------------------------------ full benchmark shapes

def _sample_rows(M, n=1500, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(range(min(64, M))) | set(range(max(0, M - 64), M))
    rows |= set(rng.integers(0, M, n).tolist())
    return sorted(rows)


@pytest.mark.slow
@pytest.mark.parametrize("name,T", [("q4_gate_up_34816x5120", 512), ("q5_down_5120x17408", 256),
                                    ("fp8_proj_5120x5120", 512)])
def test_full_size_prefill_sampled_rows(name, T):
    """Prefill-sized T on full benchmark shapes (the GEMM route): sampled rows vs the oracle."""
    fmt, M, K, _, mult = qi.CONFIGS[name]
    say(f"prefill {name} T={T}: generating")
    wl = qi.fp8_rows(name, M, K, T, mult, 1) if fmt == 8 else qi.groupwise(name, fmt, M, K, T, mult, 1)
    qm = wq.QMat(fmt, wl.codes, wl.scales)
    y = torch.full((T, M), float("nan"), device="cuda")
    wq.qmat_run(qm.handle, _x_dev(wl.x), y, T=T)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any()
    rows = _sample_rows(M, n=200, seed=2)
    worst = _check_y(y, wl, f"prefill {name} T={T}", rows=rows)
    say(f"  worst ratio {worst:.3g}")
    qm.close()


@pytest.mark.slow
@pytest.mark.parametrize("name", list(qi.CONFIGS))
def test_full_size_every_row(name):
    """Each benchmark shape at every listed T on the automatic launch plan (the one the benchmark
    times): every output element of the product against the oracle (fp64 over all rows), and
    the dequantization on ~300 sampled rows bit for bit."""
    _, _, _, Ts, _ = qi.CONFIGS[name]
    say(f"full {name}: generating")
    wl = qi.config(name)
    qm = wq.QMat(wl.fmt, wl.codes, wl.scales)
    for T in Ts:
        say(f"full {name} T={T}")
        xd = _x_dev(wl.x[:T])
        y = torch.full((T, wl.M), float("nan"), device="cuda")
        wq.qmat_run(qm.handle, xd, y, T=T)
        torch.cuda.synchronize()
        assert not torch.isnan(y).any()
        sub = qi.Workload(wl.name, wl.fmt, wl.M, wl.K, T, wl.codes, wl.scales, wl.x[:T])
        worst = _check_y(y, sub, f"{name} T={T}")
        say(f"  worst ratio {worst:.3g} over all {wl.M} rows")
        del y
    say(f"full {name}: dequant")
    drows = _sample_rows(wl.M, n=200, seed=1)
    w = qm.dequant()
    got = w[torch.tensor(drows, device="cuda")].cpu().numpy()
    del w
    if wl.fmt == 8:
        ref = oracle.dequant_fp8(wl.codes[drows], wl.scales[drows])
    else:
        ref = oracle.dequant_groupwise(qi.code_bits(wl.fmt), wl.codes[drows], wl.scales[drows])
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    qm.close()
