"""Binding of the read-stream probe (include/qmat_probe.h, libqmat_probe.so): a plain HBM read
that gives the practical bandwidth ceiling the product kernels are measured against.
Measurement support for the benchmark; argument marshalling only."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PROBE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqmat_probe.so")
SIGNATURES = {
    "qmat_probe_read_out_words": (ctypes.c_int64, [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "qmat_probe_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_void_p]),
}
# Launch shapes swept for the ceiling: (per_wave, grid_waves, unroll, waves_per_block, lds_bytes).
# Contiguous runs with one-wave workgroups held to four per compute unit by their LDS
# reservation, and grid-stride reads by 8 waves per compute unit, were the fastest in a wider
# sweep on MI355X (1 GiB: 7.0-7.1 TB/s); grid_waves -1 takes workgroup runs of per_wave chunks
# that the workgroup's waves interleave, as a head workgroup streams its 240-330 KB tile (one
# or two such workgroups per compute unit, or as many as fit); the others are common shapes for
# comparison.
SHAPES = ((256, 0, 8, 1, 40960), (64, 0, 8, 1, 40960), (64, 0, 4, 1, 20480), (256, 0, 16, 1, 0),
          (64, 0, 16, 1, 0), (0, 2048, 4, 8, 0), (0, 2048, 8, 8, 0), (0, 2048, 4, 4, 0), (32, 0, 2, 4, 0),
          (240, -1, 4, 4, 65536), (240, -1, 8, 4, 65536), (240, -1, 8, 4, 0), (240, -1, 16, 4, 0),
          (320, -1, 8, 4, 65536), (480, -1, 8, 8, 65536), (120, -1, 8, 4, 0), (240, -1, 8, 4, 40960))
_lib = None


def lib():
    """The loaded libqmat_probe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise ImportError(f"{PROBE_LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(PROBE_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def shape_name(shape) -> str:
    pw, gw, unr, wpb, lds = shape
    order = f"stride{gw}" if gw > 0 else f"block{pw}" if gw == -1 else f"run{pw}"
    return f"{order}_u{unr}_w{wpb}_lds{lds // 1024}k"


def read_out_words(nbytes: int, shape) -> int:
    pw, gw, _, wpb, _ = shape
    return int(lib().qmat_probe_read_out_words(nbytes, pw, wpb, gw))


def read(buf, nbytes: int, shape, out, stream=None) -> None:
    """Launch one read of nbytes of the device tensor buf with a launch shape (see SHAPES); out
    is a 4-byte device tensor of at least read_out_words(nbytes, shape) elements."""
    assert buf.numel() * buf.element_size() >= nbytes and out.element_size() == 4
    pw, gw, unr, wpb, lds = shape
    s: Optional[int] = None if stream is None else stream.cuda_stream
    st = lib().qmat_probe_read(buf.data_ptr(), nbytes, pw, gw, unr, wpb, lds, out.data_ptr(), out.numel(), s)
    if st != 0:
        raise RuntimeError(f"qmat_probe_read({nbytes}, {shape}) failed with status {st}")


def best_read_gbs(nbytes: int = 1 << 30, window: Optional[int] = None, reps: int = 10, shapes=SHAPES,
                  warm_s: float = 0.0, replays: int = 1):
    """Best read bandwidth (GB/s) over the launch shapes on a fresh buffer of nbytes, each timed
    as `reps` launches captured in a HIP graph and replayed (the best of `replays` timed
    replays, after replaying for warm_s seconds of wall time, so the GPU is at its steady
    clock as in the product lines).  With window set, each launch reads the next window-sized
    slice of the buffer (rotating through it, so a window smaller than the caches still streams
    from HBM).  Returns (GB/s, {shape name: GB/s})."""
    import time

    import torch
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    w = nbytes if window is None else window
    nwin = max(1, nbytes // w)
    views = [buf[i * (w // 4):(i + 1) * (w // 4)] for i in range(nwin)]
    res = {}
    for shape in shapes:
        out = torch.empty(read_out_words(w, shape), dtype=torch.int32, device="cuda")
        for i in range(2):
            read(views[i % nwin], w, shape, out)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                read(views[i % nwin], w, shape, out, stream=torch.cuda.current_stream())
        t0 = time.time()
        g.replay()
        torch.cuda.synchronize()
        while time.time() - t0 < warm_s:
            g.replay()
            torch.cuda.synchronize()
        best = 0.0
        for _ in range(max(1, replays)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            best = max(best, w * reps / (a.elapsed_time(b) * 1e-3) / 1e9)
        res[shape_name(shape)] = round(best, 1)
        del g, out
    del buf, views
    torch.cuda.empty_cache()
    return max(res.values()), res
