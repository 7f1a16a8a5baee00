"""qmat_run_static (the entry point that allocates nothing) against qmat_run on the same inputs,
through the C ABI: two calls in a row, the second with a smaller input, on matrices whose
automatic plans split K across workgroups (narrow matrices, leftover row tiles) and on the
prefill route; results must match qmat_run bit for bit (same plan, same kernels, same
summation tree) and the oracle within the product tolerance."""
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


def _x_dev(x_bits):
    return torch.from_numpy(x_bits.view(np.int16).copy()).view(torch.bfloat16).cuda()


def _case(fmt, M, K, T, seed):
    wl = qi.fp8_rows("s", M, K, T, 0.01, seed) if fmt == 8 else qi.groupwise("s", fmt, M, K, T, 0.01, seed)
    packed = torch.from_numpy(wq.qmat_pack(fmt, wl.codes, wl.scales)).cuda()
    return wl, packed


def _compare(wl, packed, T):
    x = _x_dev(wl.x[:T])
    h = wq.qmat_create(wl.fmt, wl.M, wl.K, packed)
    y_ref = torch.full((T, wl.M), float("nan"), device="cuda")
    wq.qmat_run(h, x, y_ref, T=T)
    y = torch.full((T, wl.M), float("nan"), device="cuda")
    wq.qmat_run_static(wl.fmt, wl.M, wl.K, packed, x, y, T=T)
    torch.cuda.synchronize()
    wq.qmat_destroy(h)
    assert not torch.isnan(y).any()
    assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))
    sub = qi.Workload(wl.name, wl.fmt, wl.M, wl.K, T, wl.codes, wl.scales, wl.x[:T])
    yr, A = oracle.gemv(sub.fmt, sub.codes, sub.scales, sub.x)
    ok, worst, _ = oracle.check(y.cpu().numpy(), yr, A)
    assert ok, worst


@pytest.mark.parametrize("first,second", [
    # narrow matrices: every row tile split along K (three-way trees)
    ((5, 5120, 4352, 8, 1), (5, 1000, 2048, 1, 2)),
    ((8, 5120, 5120, 16, 3), (8, 320, 640, 4, 4)),
    # more row tiles than compute units with leftover tiles split eight ways
    ((4, 17984, 1280, 4, 5), (6, 16448, 640, 1, 6)),
    # the prefill route with k splits of a narrow matrix, then a small call
    ((qi.Q8, 2048, 4096, 100, 7), (4, 700, 1024, 3, 8)),
])
def test_static_matches_run_twice(first, second):
    for fmt, M, K, T, seed in (first, second):
        say(f"static fmt={fmt} M={M} K={K} T={T}")
        wl, packed = _case(fmt, M, K, T, seed)
        _compare(wl, packed, T)


def test_static_rejects_bad_arguments():
    L = wq.lib()
    wl, packed = _case(4, 128, 256, 1, 9)
    x = _x_dev(wl.x)
    y = torch.empty((1, 128), device="cuda")
    assert L.qmat_run_static(4, 128, 256, packed.data_ptr(), packed.numel() - 1, x.data_ptr(), y.data_ptr(), 1,
                             None) == wq.QMAT_ESIZE
    assert L.qmat_run_static(3, 128, 256, packed.data_ptr(), packed.numel(), x.data_ptr(), y.data_ptr(), 1,
                             None) == wq.QMAT_EINVAL
    assert L.qmat_run_static(4, 128, 256, packed.data_ptr(), packed.numel(), x.data_ptr(), y.data_ptr(), -1,
                             None) == wq.QMAT_ESHAPE
    assert L.qmat_run_static(4, 128, 256, packed.data_ptr(), packed.numel(), x.data_ptr(), y.data_ptr(), 0,
                             None) == wq.QMAT_OK
