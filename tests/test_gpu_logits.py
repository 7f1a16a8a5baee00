"""GPU parity of the output-head epilogue (qmat_logits_*): per-token log-sum-exp and top-k
over fp32 logits, against the oracle's float64 log-sum-exp and its sort by (value descending,
row ascending).  The logits are oracle-side synthetic inputs (qmat_inputs.logits, with planted
ties), so the top-k must match bit for bit; the log-sum-exp within the fp32 evaluation bound
derived below.  An end-to-end case runs the Q6 product first and checks the epilogue against
the oracle's float64 logits within the product tolerance.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import qmat_inputs as qi
import weight_only_quant_amd as wq

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    wq.lib()


# fp32 evaluation bound of the log-sum-exp: each lane sums a few terms online, each term is
# then rescaled by at most two more exponentials (wave, block) and summed over <= 64 lanes at
# each level, each exponential and addition carrying an ulp-level error, and the last level and
# the final log are taken in double: relative error of the sum <= 64 * 2^-24 (about 4e-6),
# i.e. the same absolute error on lse, plus the final rounding of lse to fp32 (2^-24 |lse|).
def _lse_tol(ref):
    return 64 * 2.0 ** -24 + 2.0 ** -23 * np.abs(ref)


def _run(e, y, k, index=None, ldy_pad=0):
    T, M = y.shape
    yd = torch.zeros((T, M + ldy_pad), dtype=torch.float32, device="cuda")
    yd[:, :M] = torch.from_numpy(y).cuda()
    if ldy_pad:
        yd[:, M:] = 1e30  # past the row: must never be read
    lse = torch.full((T,), float("nan"), device="cuda")
    vals = torch.full((T, max(k, 1)), float("nan"), device="cuda")
    ids = torch.full((T, max(k, 1)), -7, dtype=torch.int32, device="cuda")
    idx = None if index is None else torch.from_numpy(index.astype(np.int32)).cuda()
    wq.qmat_logits_run(e, yd, k, lse=lse, top_vals=vals, top_ids=ids, index=idx)
    torch.cuda.synchronize()
    return lse.cpu().numpy(), vals.cpu().numpy()[:, :k], ids.cpu().numpy()[:, :k]


@pytest.mark.parametrize("M", [1, 5, 63, 64, 1000, 4097, 70001, 248320])
def test_lse_topk_exact_on_synthetic_logits(M):
    e = wq.qmat_logits_create(M, 16, 64)
    # k = 32 / 33: the two sides of the switch to the seeds and bounds built for large k
    for T, k, seed, pad in [(1, 1, 1, 0), (3, 7, 2, 5), (8, 20, 3, 0), (16, 64, 4, 3), (2, 0, 5, 0),
                            (4, 32, 6, 1), (5, 33, 7, 0)]:
        say(f"logits M={M} T={T} k={k} pad={pad}")
        y = qi.logits(T, M, seed=seed + M)
        lse, vals, ids = _run(e, y, k, ldy_pad=pad)
        ref = oracle.logsumexp(y)
        assert np.all(np.abs(lse.astype(np.float64) - ref) <= _lse_tol(ref)), (lse, ref)
        if k:
            rv, ri = oracle.topk(y, k)
            assert np.array_equal(vals.astype(np.float64), rv), (vals, rv)
            assert np.array_equal(ids.astype(np.int64), ri), (ids, ri)
    wq.qmat_logits_destroy(e)


def test_topk_index_map_and_all_equal_values():
    # the proposal-head shape with a row -> vocabulary id map; and a row of equal values,
    # where the order is decided by the row alone
    M = 131072
    e = wq.qmat_logits_create(M, 8, 32)
    rng = np.random.default_rng(0)
    index = rng.permutation(248320)[:M].astype(np.int64)
    y = qi.logits(4, M, seed=11)
    say("logits proposal head with index")
    lse, vals, ids = _run(e, y, 32, index=index)
    rv, ri = oracle.topk(y, 32, index)
    assert np.array_equal(vals.astype(np.float64), rv) and np.array_equal(ids.astype(np.int64), ri)
    y = np.full((2, M), 0.25, np.float32)
    lse, vals, ids = _run(e, y, 32, index=index)
    assert np.array_equal(ids[0], index[:32].astype(np.int32))
    assert abs(lse[0] - (0.25 + math.log(M))) <= _lse_tol(0.25 + math.log(M))
    wq.qmat_logits_destroy(e)


def test_repeated_calls_and_graph_replay_are_identical():
    import gc
    gc.collect()
    M, T, k = 248320, 8, 20
    e = wq.qmat_logits_create(M, T, k)
    y = torch.from_numpy(qi.logits(T, M, seed=21)).cuda()
    outs = []
    for i in range(3):
        lse = torch.empty(T, device="cuda")
        v = torch.empty((T, k), device="cuda")
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        wq.qmat_logits_run(e, y, k, lse=lse, top_vals=v, top_ids=ids)
        torch.cuda.synchronize()
        outs.append((lse.clone(), v.clone(), ids.clone()))
    for o in outs[1:]:
        assert all(torch.equal(a, b) for a, b in zip(o, outs[0]))
    lse = torch.empty(T, device="cuda")
    v = torch.empty((T, k), device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wq.qmat_logits_run(e, y, k, lse=lse, top_vals=v, top_ids=ids)
    for i in range(3):
        lse.fill_(float("nan"))
        ids.fill_(-5)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lse, outs[0][0]) and torch.equal(v, outs[0][1]) and torch.equal(ids, outs[0][2]), i
        wq.qmat_logits_run(e, y, k, lse=torch.empty(T, device="cuda"), top_vals=torch.empty((T, k), device="cuda"),
                           top_ids=torch.empty((T, k), dtype=torch.int32, device="cuda"))  # eager work between
        torch.cuda.synchronize()
    del g
    wq.qmat_logits_destroy(e)


def test_head_product_then_epilogue_end_to_end():
    # Q6 head-like matrix: product on the GPU, epilogue on its logits, against the oracle's
    # float64 logits.  lse is 1-Lipschitz in the max norm, so |lse - lse_ref| <= max_i tol_i
    # (the product tolerance) plus the fp32 evaluation bound; each returned value is the
    # GPU logit of the returned row, within tol of the oracle's; and no row left out beats the
    # smallest returned one by more than twice the tolerance.
    M, K, T, k = 9000, 512, 8, 16
    wl = qi.groupwise("h", 6, M, K, T, 0.005, 5)
    qm = wq.QMat(6, wl.codes, wl.scales)
    xd = torch.from_numpy(wl.x.view(np.int16).copy()).view(torch.bfloat16).cuda()
    y = qm.run(xd)
    e = wq.qmat_logits_create(M, T, k)
    lse = torch.empty(T, device="cuda")
    v = torch.empty((T, k), device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wq.qmat_logits_run(e, y, k, lse=lse, top_vals=v, top_ids=ids)
    torch.cuda.synchronize()
    y_ref, A = oracle.gemv(6, wl.codes, wl.scales, wl.x)
    tol = oracle.REL_TOL * A + oracle.ABS_TOL
    lse_ref = oracle.logsumexp(y_ref)
    got = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - lse_ref) <= tol.max(axis=1) + _lse_tol(lse_ref))
    yg = y.cpu().numpy()
    vv, ii = v.cpu().numpy(), ids.cpu().numpy()
    for t in range(T):
        assert len(set(ii[t].tolist())) == k
        assert np.array_equal(vv[t], yg[t, ii[t]])
        assert np.all(np.abs(vv[t] - y_ref[t, ii[t]]) <= tol[t, ii[t]])
        rest = np.setdiff1d(np.arange(M), ii[t])
        assert y_ref[t, rest].max() <= y_ref[t, ii[t]].min() + 2 * tol[t].max()
    wq.qmat_logits_destroy(e)
    qm.close()


def test_epilogue_argument_errors():
    e = wq.qmat_logits_create(100, 4, 8)
    y = torch.zeros((4, 100), device="cuda")
    v = torch.empty((4, 8), device="cuda")
    ids = torch.empty((4, 8), dtype=torch.int32, device="cuda")
    for kw, status in [(dict(k=9), wq.QMAT_ESHAPE), (dict(k=-1), wq.QMAT_ESHAPE), (dict(k=2, T=5), wq.QMAT_ESHAPE)]:
        with pytest.raises(wq.QmatError) as err:
            wq.qmat_logits_run(e, y, top_vals=v, top_ids=ids, **kw)
        assert err.value.status == status, kw
    with pytest.raises(wq.QmatError) as err:
        wq.qmat_logits_run(e, y, 2)  # k > 0 without outputs
    assert err.value.status == wq.QMAT_EINVAL
    assert wq.lib().qmat_logits_run(e, y.data_ptr(), 50, 1, 2, None, None, v.data_ptr(), ids.data_ptr(),
                                    None) == wq.QMAT_ESHAPE  # ldy < M
    wq.qmat_logits_run(e, y, 0, T=0)  # no-op
    wq.qmat_logits_destroy(e)
    for args in [(0, 4, 8), (100, 0, 8), (100, 17, 8), (100, 4, 65)]:
        with pytest.raises(wq.QmatError) as err:
            wq.qmat_logits_create(*args)
        assert err.value.status == wq.QMAT_ESHAPE, args


# ------------------------------------------------------------------ product and epilogue in one call

def _head(fmt, M, K, T, seed, exact=False):
    if exact:
        # every product and partial sum exact in fp32 (small integer activations, power-of-two
        # scales, integer-valued E4M3 bytes): the logits equal the oracle's float64 ones, with
        # many equal values among the largest
        rng = np.random.default_rng(seed)
        x = torch.from_numpy(rng.integers(-4, 5, (T, K)).astype(np.float32)).to(torch.bfloat16)
        x_bits = x.view(torch.int16).numpy().view(np.uint16)
        if fmt == 8:
            ints = rng.integers(-16, 17, (M, K)).astype(np.float32)
            codes = torch.from_numpy(ints).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            scales = (2.0 ** rng.integers(-6, 3, M)).astype(np.float32)
        else:
            b = qi.code_bits(fmt)
            codes = rng.integers(-(1 << (b - 1)), 1 << (b - 1), (M, K)).astype(np.int8)
            sg = np.where(rng.random((M, K // 64)) < 0.5, -1.0, 1.0)
            scales = (sg * 2.0 ** rng.integers(-2, 2, (M, K // 64))).astype(np.float16).view(np.uint16)
        return qi.Workload("exact", fmt, M, K, T, codes, scales, x_bits)
    if fmt == 8:
        return qi.fp8_rows("h", M, K, T, 0.01, seed)
    return qi.groupwise("h", fmt, M, K, T, 0.005, seed)


def _both(qm, e, xd, T, k, index=None, with_y=True):
    y = torch.full((T, qm.M), float("nan"), device="cuda") if with_y else None
    lse = torch.full((T,), float("nan"), device="cuda")
    vals = torch.full((T, max(k, 1)), float("nan"), device="cuda")
    ids = torch.full((T, max(k, 1)), -7, dtype=torch.int32, device="cuda")
    wq.qmat_run_logits(qm.handle, e, xd[:T], k, y=y, lse=lse, top_vals=vals, top_ids=ids, index=index, T=T)
    torch.cuda.synchronize()
    return y, lse.cpu().numpy(), vals.cpu().numpy()[:, :k], ids.cpu().numpy()[:, :k]


# head-shaped matrices (many row tiles, no split of K), ragged last tiles included
HEAD_SHAPES = [(6, 131072 + 37, 640), (8, 131072, 512), (qi.Q8, 140000, 384), (4, 2049 * 64 - 63, 256)]


@pytest.mark.parametrize("fmt,M,K", HEAD_SHAPES)
def test_run_logits_matches_product_then_pass(fmt, M, K):
    """qmat_run_logits on a head-shaped matrix: y bit for bit qmat_run's; top-k identical to the
    separate epilogue call on that y and to the oracle's sort of it; lse within the fp32
    evaluation bound of the oracle's float64 log-sum-exp of that y; the same outputs without y."""
    wl = _head(fmt, M, K, 16, 30 + fmt)
    qm = wq.QMat(fmt, wl.codes, wl.scales)
    xd = torch.from_numpy(wl.x.view(np.int16).copy()).view(torch.bfloat16).cuda()
    e = wq.qmat_logits_create(M, 16, 64)
    rng = np.random.default_rng(M)
    index = rng.permutation(2 * M)[:M].astype(np.int32) if fmt == qi.Q8 else None
    idx = None if index is None else torch.from_numpy(index).cuda()
    for T, k in [(1, 20), (2, 1), (3, 0), (8, 20), (10, 64), (16, 7)]:
        say(f"run_logits fmt={fmt} M={M} T={T} k={k}")
        y, lse, vals, ids = _both(qm, e, xd, T, k, idx)
        y_run = qm.run(xd[:T])
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y_run.view(torch.int32))
        yg = y.cpu().numpy()
        ref = oracle.logsumexp(yg)
        assert np.all(np.abs(lse.astype(np.float64) - ref) <= _lse_tol(ref)), (lse, ref)
        if k:
            rv, ri = oracle.topk(yg, k, None if index is None else index.astype(np.int64))
            assert np.array_equal(vals.astype(np.float64), rv), (vals, rv)
            assert np.array_equal(ids.astype(np.int64), ri), (ids, ri)
            lse2, vals2, ids2 = _run(e, yg, k, index=index)
            assert np.array_equal(vals, vals2) and np.array_equal(ids, ids2)
        _, lse3, vals3, ids3 = _both(qm, e, xd, T, k, idx, with_y=False)
        assert np.array_equal(lse3.view(np.int32), lse.view(np.int32))
        assert np.array_equal(vals3, vals) and np.array_equal(ids3, ids)
    wq.qmat_logits_destroy(e)
    qm.close()


@pytest.mark.parametrize("fmt", [6, 8])
def test_run_logits_bit_exact_on_exact_inputs(fmt):
    """Exact-arithmetic inputs (logits with many equal values, also across row blocks): the
    top-k equals the oracle's sort of its float64 logits, ties ordered by row."""
    M, K = 131072 + 64 * 3, 256
    for T, k in [(1, 64), (8, 20), (16, 5)]:
        wl = _head(fmt, M, K, T, 50 + T, exact=True)
        qm = wq.QMat(fmt, wl.codes, wl.scales)
        xd = torch.from_numpy(wl.x.view(np.int16).copy()).view(torch.bfloat16).cuda()
        e = wq.qmat_logits_create(M, T, k)
        say(f"run_logits exact fmt={fmt} T={T} k={k}")
        _, lse, vals, ids = _both(qm, e, xd, T, k, with_y=False)
        y_ref, _ = oracle.gemv(fmt, wl.codes, wl.scales, wl.x)
        rv, ri = oracle.topk(y_ref, k)
        assert np.array_equal(vals.astype(np.float64), rv) and np.array_equal(ids.astype(np.int64), ri)
        ref = oracle.logsumexp(y_ref)
        assert np.all(np.abs(lse.astype(np.float64) - ref) <= _lse_tol(ref))
        wq.qmat_logits_destroy(e)
        qm.close()


def test_run_logits_end_to_end_and_graph_replay():
    """The Q6 head shape at T = 8: the outputs against the oracle's float64 logits (as in the
    separate-pass end-to-end test), repeated calls identical, and graph replays of the product
    and both epilogue kernels identical to the eager result."""
    import gc
    gc.collect()
    M, K, T, k = 248320, 512, 8, 20
    wl = qi.groupwise("h", 6, M, K, T, 0.005, 77)
    qm = wq.QMat(6, wl.codes, wl.scales)
    xd = torch.from_numpy(wl.x.view(np.int16).copy()).view(torch.bfloat16).cuda()
    e = wq.qmat_logits_create(M, T, k)
    y, lse, vals, ids = _both(qm, e, xd, T, k)
    y_ref, A = oracle.gemv(6, wl.codes, wl.scales, wl.x)
    tol = oracle.REL_TOL * A + oracle.ABS_TOL
    lse_ref = oracle.logsumexp(y_ref)
    assert np.all(np.abs(lse.astype(np.float64) - lse_ref) <= tol.max(axis=1) + _lse_tol(lse_ref))
    yg = y.cpu().numpy()
    for t in range(T):
        assert len(set(ids[t].tolist())) == k
        assert np.array_equal(vals[t], yg[t, ids[t]])
        assert np.all(np.abs(vals[t] - y_ref[t, ids[t]]) <= tol[t, ids[t]])
        rest = np.setdiff1d(np.arange(M), ids[t])
        assert y_ref[t, rest].max() <= y_ref[t, ids[t]].min() + 2 * tol[t].max()
    for i in range(2):
        _, lse2, vals2, ids2 = _both(qm, e, xd, T, k, with_y=False)
        assert np.array_equal(lse2.view(np.int32), lse.view(np.int32)) and np.array_equal(vals2, vals)
        assert np.array_equal(ids2, ids)
    lse_d = torch.empty(T, device="cuda")
    v_d = torch.empty((T, k), device="cuda")
    i_d = torch.empty((T, k), dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wq.qmat_run_logits(qm.handle, e, xd, k, lse=lse_d, top_vals=v_d, top_ids=i_d)
    for i in range(4):
        lse_d.fill_(float("nan"))
        i_d.fill_(-5)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(lse_d.cpu().numpy().view(np.int32), lse.view(np.int32)), i
        assert np.array_equal(v_d.cpu().numpy(), vals) and np.array_equal(i_d.cpu().numpy(), ids), i
        _both(qm, e, xd, T, k, with_y=False)  # eager work between replays
    del g
    wq.qmat_logits_destroy(e)
    qm.close()


def test_run_logits_on_a_split_plan_and_errors():
    """A matrix whose plan splits K (the exchange-tree reduction runs first), with or without y;
    and the argument checks."""
    M, K, T, k = 5000, 4352, 4, 16
    wl = qi.groupwise("s", 5, M, K, T, 0.01, 88)
    qm = wq.QMat(5, wl.codes, wl.scales)
    assert wq.qmat_get_plan(qm.handle, T).splits > 1
    xd = torch.from_numpy(wl.x.view(np.int16).copy()).view(torch.bfloat16).cuda()
    e = wq.qmat_logits_create(M, T, k)
    y, lse, vals, ids = _both(qm, e, xd, T, k)
    yg = y.cpu().numpy()
    rv, ri = oracle.topk(yg, k)
    assert np.array_equal(vals.astype(np.float64), rv) and np.array_equal(ids.astype(np.int64), ri)
    _, lse2, vals2, ids2 = _both(qm, e, xd, T, k, with_y=False)
    assert np.array_equal(vals2, vals) and np.array_equal(ids2, ids)
    L = wq.lib()
    e2 = wq.qmat_logits_create(M + 1, T, k)
    assert L.qmat_run_logits(qm.handle, e2, xd.data_ptr(), None, T, k, None, None, vals2.ctypes.data, None,
                             None) == wq.QMAT_ESHAPE
    assert L.qmat_run_logits(qm.handle, e, xd.data_ptr(), None, T, k + 1, None, None, None, None,
                             None) == wq.QMAT_ESHAPE
    assert L.qmat_run_logits(qm.handle, e, xd.data_ptr(), None, T, k, None, None, None, None, None) == wq.QMAT_EINVAL
    assert L.qmat_run_logits(None, e, xd.data_ptr(), None, T, k, None, None, None, None, None) == wq.QMAT_EINVAL
    assert L.qmat_run_logits(qm.handle, e, xd.data_ptr(), None, 0, k, None, None, None, None, None) == wq.QMAT_OK
    wq.qmat_logits_destroy(e2)
    wq.qmat_logits_destroy(e)
    qm.close()


@pytest.mark.parametrize("n_equal", [63, 300])
def test_candidate_overflow_paths(n_equal):
    """Logits that overflow the kernels' candidate buffers: every block of 2048 rows holds
    n_equal rows of one equal top value.  With 63, at k = 64 the merge keeps 2521 candidates
    (more than its 1024: its sorting-network path); with 300 the block pass keeps 300 at k = 20
    and at k = 64 (more than its 256: its sorting-network path).  The top-k must still equal
    the oracle's sort, ties by row."""
    M, T, k = 40 * 2048, 2, 64  # 40 whole blocks of 2048 rows
    rng = np.random.default_rng(4)
    y = rng.standard_normal((T, M)).astype(np.float32)
    for t in range(T):
        for b0 in range(0, M, 2048):
            n = min(2048, M - b0)
            rows = b0 + rng.choice(n, size=min(n_equal, n), replace=False)
            y[t, rows] = 100.0 + t
    e = wq.qmat_logits_create(M, T, k)
    say(f"logits candidate overflow, {n_equal} equal values per block")
    lse, vals, ids = _run(e, y, k)
    rv, ri = oracle.topk(y, k)
    assert np.array_equal(vals.astype(np.float64), rv) and np.array_equal(ids.astype(np.int64), ri)
    ref = oracle.logsumexp(y)
    assert np.all(np.abs(lse.astype(np.float64) - ref) <= _lse_tol(ref))
    lse2, vals2, ids2 = _run(e, y, 20)
    rv, ri = oracle.topk(y, 20)
    assert np.array_equal(vals2.astype(np.float64), rv) and np.array_equal(ids2.astype(np.int64), ri)
    wq.qmat_logits_destroy(e)


def test_many_rounds_per_block():
    """4M rows: 512 blocks of 8192 rows, four rounds of loads per block (each lane's running
    sum carried across rounds); top-k and log-sum-exp against the oracle as above."""
    M, T, k = 4 << 20, 2, 20
    e = wq.qmat_logits_create(M, T, k)
    say("logits many rounds per block")
    y = qi.logits(T, M, seed=9)
    lse, vals, ids = _run(e, y, k)
    ref = oracle.logsumexp(y)
    assert np.all(np.abs(lse.astype(np.float64) - ref) <= _lse_tol(ref)), (lse, ref)
    rv, ri = oracle.topk(y, k)
    assert np.array_equal(vals.astype(np.float64), rv) and np.array_equal(ids.astype(np.int64), ri)
    wq.qmat_logits_destroy(e)
