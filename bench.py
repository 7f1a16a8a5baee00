"""Benchmark of the weight-only quantized small-T product on one MI355X.

A step is one qmat_run call (the whole product: stream packed codes and scales, unpack,
dot products, group scales, reductions, write y) on resident device buffers.  The headline
workload is the Q4 fused MLP gate+up projection (two 17408 x 5120 matrices as one
M=34816, K=5120 matrix) at T=1; the other benchmark shapes (Q6 vocab head, Q5 down
projection with split-K, FP8 row-scaled head and projection, the 8-bit heads, the small Q4
case) at each of their token counts are reported in "extra", and so is the gate+up matrix on the
explicit offset-operand route (QMAT_ROUTE_MFMA_OFFSET, "_offset_route").

Throughput is algorithmic bytes (packed codes + scales read once, x read, y written) per
second.  Matrices smaller than 512 MB rotate over enough device copies to exceed 512 MB so
the 256 MB Infinity Cache cannot serve them.  Inputs are seeded synthetic data.

Timing protocol.  Every timed region follows a time-based warm-up on its own workload (the
GPU runs that workload for a fixed wall time first, whatever --warmup says, so that clocks
and caches are at steady state after host-side setup).  The headline line times exactly
--steps launches captured in one HIP graph, once (value and ms_per_step, the launch of the
graph included); its roofline divides the bytes by the kernel's marginal time per launch, from
a graph of twice the launches timed against it.  The other decode lines run in two rounds,
the second in reverse order (every pair of lines is timed A-B-B-A), each round timing three
replays of a graph of at least 50 launches; the reported time is the median over all
replays, with the per-round medians beside it.  Every decode line also reports the event time
of single eager launches, each alone on an idle stream (median, 10th and 90th percentile of
40).  All decode lines run before the epilogue, prefill and read-probe lines.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "weight GB/s & % HBM peak, Q4 MLP and Q6 vocab head at T=1 and T=8; µs/call"
HBM_PEAK_GBS = 8000.0
PRIMARY = ("q4_gate_up_34816x5120", 1)
ROTATE_BYTES = 512 << 20
PREFILL_T = (512, 2048)                      # prefill chunk sizes timed on the GEMM route
PROBE_WARM_S = 0.3  # wall time each read-probe shape replays before it is timed (best of 3 replays)
PREFILL_SHAPES = ("q5_down_5120x17408", "fp8_proj_5120x5120")
WARM_S = 0.25            # wall time each decode line runs before it is timed
WARM_HEADLINE_S = 1.0    # the same for the headline line
MIN_CALLS = 50           # launches per timed replay on the decode lines
REPLAYS = 3              # timed replays per line and round
ROUNDS = 2               # the second in reverse order


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def alg_bytes(fmt, M, K, T):
    """Packed weight information (codes + scales, each read once) + x read + y written."""
    import qmat_inputs as qi
    if fmt == 8:
        w = M * K + 4 * M
    else:
        w = M * K * qi.code_bits(fmt) // 8 + 2 * M * (K // 64)
    return w + 2 * T * K + 4 * T * M


class Resident:
    """One workload packed and resident on the GPU, with rotation copies."""

    def __init__(self, name, seed=0):
        import torch
        import qmat_inputs as qi
        import weight_only_quant_amd as wq
        self.name = name
        t0 = time.time()
        wl = qi.config(name, seed=seed)
        self.wl = wl
        packed = wq.qmat_pack(wl.fmt, wl.codes, wl.scales)
        dev = torch.from_numpy(packed).cuda()
        n = max(1, math.ceil(ROTATE_BYTES / packed.size))
        self.copies = [dev] + [dev.clone() for _ in range(n - 1)]
        self.handles = [wq.qmat_create(wl.fmt, wl.M, wl.K, c) for c in self.copies]
        self.x = torch.from_numpy(wl.x.view(np.int16).copy()).view(torch.bfloat16).cuda()
        self.y = torch.empty((wl.T, wl.M), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        log(f"[bench] {name}: M={wl.M} K={wl.K} fmt={wl.fmt} packed {packed.size / 1e6:.1f} MB x{len(self.copies)} "
            f"copies, setup {time.time() - t0:.1f}s")

    def close(self):
        import weight_only_quant_amd as wq
        for h in self.handles:
            wq.qmat_destroy(h)
        self.handles = []
        self.copies = []


class Timed:
    """n launches of one decode workload captured in one HIP graph (rotating over the
    resident copies), replayed on the current stream; route 0 is the automatic route."""

    def __init__(self, res, T, n, route=0):
        import gc
        import torch
        import weight_only_quant_amd as wq
        self.res, self.T, self.n = res, T, n
        x, y = res.x[:T], res.y[:T]
        hs = res.handles
        gc.collect()
        torch.cuda.synchronize()
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g):
            for i in range(n):
                if route:
                    wq.qmat_run_ex(hs[i % len(hs)], x, y, T, route=route)
                else:
                    wq.qmat_run(hs[i % len(hs)], x, y, T=T)
        torch.cuda.synchronize()

    def warm(self, seconds):
        """Replay until `seconds` of wall time have passed (at least twice)."""
        import torch
        t0, k = time.time(), 0
        while k < 2 or time.time() - t0 < seconds:
            self.g.replay()
            k += 1
            if k % 4 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()

    def time_once(self):
        """One replay bracketed by events on the replay stream: ms per launch."""
        import torch
        stream = torch.cuda.current_stream()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        self.g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / self.n

    def close(self):
        del self.g


def qmat_packed_size(name):
    """Packed bytes (codes + scales) of a benchmark workload."""
    import qmat_inputs as qi
    import weight_only_quant_amd as wq
    c = qi.CONFIGS[name]
    return wq.qmat_packed_bytes(c[0], c[1], c[2])


def plan_str(res, T, route=0):
    import weight_only_quant_amd as wq
    p = wq.qmat_get_plan(res.handles[0], T, route)
    tail = f" tail_tiles={p.tail_tiles} tail_splits={p.tail_splits}" if p.tail_tiles else ""
    tiles = f" tiles={p.tiles}" if p.tiles > 1 else ""
    name = {wq.QMAT_ROUTE_VALU: "valu", wq.QMAT_ROUTE_MFMA_OFFSET: "mfma-offset"}.get(p.route, "mfma")
    return f"{name} depth={p.depth} waves={p.waves} splits={p.splits}{tail}{tiles}"


def line(res, T, us_list, per_round, single, route=0):
    """A decode line from per-launch times (µs) of all timed replays, with the single-launch
    event times beside it."""
    wl = res.wl
    ab = alg_bytes(wl.fmt, wl.M, wl.K, T)
    us = float(np.median(us_list))
    return {"us_per_call": round(us, 3), "us_min": round(min(us_list), 3), "us_max": round(max(us_list), 3),
            "us_round_medians": [round(v, 3) for v in per_round], "timed_replays": len(us_list),
            "GBps": round(ab / us / 1e3, 1), "pct_hbm_peak": round(100 * ab / us / 1e3 / HBM_PEAK_GBS, 2),
            "bytes": ab, "plan": plan_str(res, T, route), "single_launch_us": single}


SINGLE_WARM = 20   # eager launches before the single-launch timings of a line
SINGLE_N = 40      # single launches timed per line


def single_launch(res, T, route=0):
    """Each of SINGLE_N eager launches alone on an idle stream, bracketed by events and
    synchronized after: median, 10th and 90th percentile of the event time (µs).  This is the
    latency of one call on its own (dispatch and ramp-up included), beside the back-to-back
    average of the graph replays."""
    import torch
    import weight_only_quant_amd as wq
    hs, x, y = res.handles, res.x[:T], res.y[:T]
    stream = torch.cuda.current_stream()
    def run(h):
        if route:
            wq.qmat_run_ex(h, x, y, T, route=route)
        else:
            wq.qmat_run(h, x, y, T=T)

    for i in range(SINGLE_WARM):
        run(hs[i % len(hs)])
    torch.cuda.synchronize()
    us = []
    for i in range(SINGLE_N):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run(hs[(SINGLE_WARM + i) % len(hs)])
        b.record(stream)
        torch.cuda.synchronize()
        us.append(a.elapsed_time(b) * 1e3)
    p10, p50, p90 = np.percentile(us, [10, 50, 90])
    return {"median": round(float(p50), 3), "p10": round(float(p10), 3), "p90": round(float(p90), 3), "n": SINGLE_N}


def measure_decode(lines, steps):
    """Every (Resident, T, route) in `lines`, ROUNDS rounds alternating forward / reverse order;
    each round warms the line for WARM_S and times REPLAYS replays of a graph of >= MIN_CALLS
    launches."""
    times = {i: [] for i in range(len(lines))}
    rounds = {i: [] for i in range(len(lines))}
    for r in range(ROUNDS):
        order = range(len(lines)) if r % 2 == 0 else reversed(range(len(lines)))
        for i in order:
            res, T, route = lines[i]
            # every rotation copy at least once per replay (the small matrix has thousands)
            n = max(MIN_CALLS, steps, min(len(res.handles), 4096))
            tm = Timed(res, T, n, route)
            tm.warm(WARM_S)
            us = [tm.time_once() * 1e3 for _ in range(REPLAYS)]
            tm.close()
            times[i] += us
            rounds[i].append(float(np.median(us)))
            log(f"[bench] round {r} {res.name} T={T}: {np.median(us):.3f} us/call")
    single = {}
    for i, (res, T, route) in enumerate(lines):
        single[i] = single_launch(res, T, route)
        log(f"[bench] single launch {res.name} T={T} route={route}: {single[i]}")
    return {i: line(lines[i][0], lines[i][1], times[i], rounds[i], single[i], lines[i][2]) for i in range(len(lines))}


def measure_epilogue(res, T, k, warm_s=WARM_S, n=MIN_CALLS, with_product=False):
    """The output-head epilogue (per-token log-sum-exp and top-k) on the logits the head product
    left in res.y, graph-replayed after a time-based warm-up; bytes are the logits read.  With
    with_product, the head product and the epilogue in one call (qmat_run_logits, logits kept in
    the epilogue's own buffer); bytes are then the packed matrix and the logits written and read."""
    import torch
    import weight_only_quant_amd as wq
    M = res.wl.M
    e = wq.qmat_logits_create(M, T, k)
    y = res.y[:T]
    lse = torch.empty(T, device="cuda")
    v = torch.empty((T, k), device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")

    def call(i):
        if with_product:
            h = res.handles[i % len(res.handles)]
            wq.qmat_run_logits(h, e, res.x[:T], k, lse=lse, top_vals=v, top_ids=ids)
        else:
            wq.qmat_logits_run(e, y, k, lse=lse, top_vals=v, top_ids=ids)

    call(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            call(i)
    t0 = time.time()
    while time.time() - t0 < warm_s:
        g.replay()
        torch.cuda.synchronize()
    us = []
    for _ in range(REPLAYS):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        us.append(a.elapsed_time(b) / n * 1e3)
    del g
    wq.qmat_logits_destroy(e)
    nb = T * M * 4 + (res.copies[0].numel() + T * res.wl.K * 2 + T * M * 4 if with_product else 0)
    u = float(np.median(us))
    return {"us_per_call": round(u, 3), "GBps": round(nb / u / 1e3, 1), "bytes": nb, "k": k}


def measure_prefill(res, T, calls=20, warm_s=WARM_S, reference=False):
    """A prefill-sized product (the GEMM route) on the resident matrix with T synthetic bf16
    activation rows, after a time-based warm-up; throughput in TFLOP/s (2 T M K per call)."""
    import torch
    import weight_only_quant_amd as wq
    wl = res.wl
    g = torch.Generator(device="cuda")
    g.manual_seed(T)
    x = torch.randn((T, wl.K), generator=g, device="cuda").to(torch.bfloat16)
    y = torch.empty((T, wl.M), device="cuda")
    hs = res.handles

    def timed(fn):
        t0, i = time.time(), 0
        while i < 3 or time.time() - t0 < warm_s:
            fn(i)
            i += 1
            torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(calls):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / calls * 1e3

    us = timed(lambda i: wq.qmat_run(hs[i % len(hs)], x, y, T=T))
    tf = 2.0 * T * wl.M * wl.K / us / 1e6
    out = {"us_per_call": round(us, 2), "TFLOPs": round(tf, 1), "pct_bf16_mfma_peak": round(100 * tf / 2500.0, 2),
           "route": "gemm"}
    if reference:
        # context, not the product: the vendor bf16 GEMM (torch.matmul -> hipBLASLt) on an
        # unquantized bf16 weight of the same shape, the practical matrix-core rate on this GPU
        w = torch.randn((wl.M, wl.K), generator=g, device="cuda").to(torch.bfloat16)
        ref_us = timed(lambda i: torch.matmul(x, w.t()))
        out["bf16_vendor_gemm_us"] = round(ref_us, 2)
        out["bf16_vendor_gemm_TFLOPs"] = round(2.0 * T * wl.M * wl.K / ref_us / 1e6, 1)
        out["pct_of_vendor_bf16_gemm"] = round(100 * ref_us / us, 1)
        del w
    del x, y
    return out


def cpu_baseline(wl, T, target_s=12.0):
    """The CPU oracle (as it stands) on a bounded sample of the same workload: whole passes
    over all rows (or a row subset when one pass would exceed the budget), repeated until
    about target_s seconds of CPU work have run."""
    import oracle
    threads = min(os.cpu_count() or 1, 16)
    x = wl.x[:T]
    probe = np.arange(min(wl.M, 512))
    t0 = time.time()
    oracle.gemv(wl.fmt, wl.codes, wl.scales, x, rows=probe, nthreads=threads)
    per_row_s = max(time.time() - t0, 1e-6) / len(probe)
    n = int(min(wl.M, max(512, target_s / per_row_s)))
    rows = None if n == wl.M else np.linspace(0, wl.M - 1, n).astype(np.int64)
    passes, t0 = 0, time.time()
    while True:
        oracle.gemv(wl.fmt, wl.codes, wl.scales, x, rows=rows, nthreads=threads)
        passes += 1
        if time.time() - t0 >= target_s:
            break
    dt = time.time() - t0
    per_row = alg_bytes(wl.fmt, 1, wl.K, 0)
    gbs = passes * (n * per_row + 2 * T * wl.K + 4 * T * n) / dt / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{passes} pass(es) over {n} of {wl.M} rows of {wl.name} at T={T} in {dt:.1f} s "
                      f"(fp64 scalar C, {threads} threads)"}


def read_ceilings(window_bytes, big_bytes):
    """Practical read-bandwidth ceilings from the read-stream probe (libqmat_probe.so, a plain
    16-byte-per-lane nontemporal read; best of its launch shapes): over a buffer at least as
    large as the largest benchmark matrix, and over windows of the headline matrix's size
    rotated through 1 GiB (so each read streams from HBM, as the rotated weight copies do)."""
    from weight_only_quant_amd import probe
    big, big_shapes = probe.best_read_gbs(big_bytes, warm_s=PROBE_WARM_S, replays=3)
    w = window_bytes // 1024 * 1024
    win, _ = probe.best_read_gbs(1 << 30, window=w, reps=100, warm_s=PROBE_WARM_S, replays=3)
    return {"GBps_big": big, "big_bytes": big_bytes, "shapes_big": big_shapes, "GBps_window": win, "window_bytes": w}


def read_probe_window(window_bytes):
    """Best plain-read rate (GB/s) over windows of window_bytes rotated through 1 GiB."""
    from weight_only_quant_amd import probe
    return probe.best_read_gbs(1 << 30, window=window_bytes, reps=100, warm_s=PROBE_WARM_S, replays=3)


def cpu_context(target_s=1.0):
    """The host CPU model and the oracle's single-thread time on the small Q4 case (256 x 1024,
    T = 1), the one the measurement plan times on one core."""
    import oracle
    import qmat_inputs as qi
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    wl = qi.config("q4_small_256x1024")
    n, t0 = 0, time.time()
    while True:
        oracle.gemv(wl.fmt, wl.codes, wl.scales, wl.x[:1], nthreads=1)
        n += 1
        if time.time() - t0 >= target_s:
            break
    us = (time.time() - t0) / n * 1e6
    return {"cpu_model": model, "host_threads": os.cpu_count(),
            "q4_small_256x1024_T1_single_thread_us": round(us, 1)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5,
                    help="graph replays after the time-based warm-up (which always runs)")
    ap.add_argument("--primary-only", action="store_true", help="skip the other benchmark shapes")
    ap.add_argument("--only", default=None, help="comma-separated config names for the extra shapes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 256 MiB device copy (known bytes) for scaling PMC byte counters")
    ap.add_argument("--eager-only", action="store_true",
                    help="time eager stream launches only (no graph replay), for counter profilers that "
                         "serialize dispatches")
    ap.add_argument("--profile-lines", default=None,
                    help="only run these decode lines (name:T,...), --warmup then --steps eager launches "
                         "each, for counter profilers")
    ap.add_argument("--route", choices=("auto", "valu", "mfma", "offset"), default="auto",
                    help="small-T route of the --profile-lines launches")
    args = ap.parse_args()
    if args.gpus != 1:
        log("bench.py: this benchmark runs on one GPU only: the product shards by rows with no "
            "collective, so a multi-GPU figure would be N independent copies of this one; --gpus must be 1")
        sys.exit(2)

    import torch
    import qmat_inputs as qi
    import weight_only_quant_amd as wq
    if args.copy_calibration:
        src = torch.ones((64 << 20,), dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {src.numel() * 4} bytes x5")
        return
    if not os.path.exists(wq.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wq.lib()
    if args.profile_lines:
        route = {"auto": wq.QMAT_ROUTE_AUTO, "valu": wq.QMAT_ROUTE_VALU, "mfma": wq.QMAT_ROUTE_MFMA,
                 "offset": wq.QMAT_ROUTE_MFMA_OFFSET}[args.route]
        for item in args.profile_lines.split(","):
            pname, pT = item.split(":")
            pT = int(pT)
            r = Resident(pname)
            hs = r.handles
            for i in range(args.warmup + args.steps):
                wq.qmat_run_ex(hs[i % len(hs)], r.x[:pT], r.y[:pT], T=pT, route=route)
            torch.cuda.synchronize()
            log(f"[bench] profiled {pname} T={pT} route={args.route}: {args.warmup} + {args.steps} launches, "
                f"plan {plan_str(r, pT, route)}")
            r.close()
        return

    name, T = PRIMARY
    res = Resident(name)
    wl = res.wl
    ab = alg_bytes(wl.fmt, wl.M, wl.K, T)
    if args.eager_only:
        hs = res.handles
        for i in range(args.warmup):
            wq.qmat_run(hs[i % len(hs)], res.x[:T], res.y[:T], T=T)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(args.steps):
            wq.qmat_run(hs[i % len(hs)], res.x[:T], res.y[:T], T=T)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / args.steps
        extra_replays = []
        launch_us = ms * 1e3
    else:
        # exactly --steps launches in one graph: time-based warm-up, --warmup more replays,
        # then one timed replay (the contract's timed region)
        tm = Timed(res, T, args.steps)
        tm.warm(WARM_HEADLINE_S)
        for _ in range(args.warmup):
            tm.g.replay()
        ms = tm.time_once()
        # more replays of the same graph, reported beside the line (not the headline value)
        extra_replays = [round(tm.time_once() * 1e3, 3) for _ in range(5)]
        tm.close()
        # the kernel's own time per launch: a graph of twice the launches against this one
        # (medians of 6 replays each), which cancels the one-off cost of launching a graph
        t1 = float(np.median([ms * 1e3] + extra_replays)) * args.steps
        tm2 = Timed(res, T, 2 * args.steps)
        tm2.warm(WARM_S)
        t2 = float(np.median([tm2.time_once() * 1e3 for _ in range(6)])) * 2 * args.steps
        tm2.close()
        launch_us = (t2 - t1) / args.steps
    value = ab / (ms * 1e-3) / 1e9
    log(f"[bench] {name} T={T}: {ms * 1e3:.3f} us/call, {value:.1f} GB/s; more replays {extra_replays}")
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{name}_T{T}", "format": "Q4 groupwise (64-weight groups, FP16 scales)",
                   "M": wl.M, "K": wl.K, "T": T, "x": "bf16", "y": "fp32", "global_batch": T,
                   "parallelism": "single-gpu", "rotation_copies": len(res.copies),
                   "launch": "eager stream launches" if args.eager_only else
                             "--steps launches captured in one HIP graph, one timed replay after a "
                             f"{WARM_HEADLINE_S:.1f} s time-based warm-up",
                   "plan": plan_str(res, T)},
        # one launch per step.  ms_per_step (and value) include the one-off cost of launching
        # the graph of --steps launches; achieved divides the bytes by the kernel's marginal
        # time per launch (a 2 x --steps graph against the --steps one, graph replays only),
        # the duration a kernel trace of this command reports
        "roofline": {"bound": "hbm", "achieved": round(ab / (launch_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ab / (launch_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"{name}_T{T}"),
                     "launch_us_mean": round(launch_us, 3), "bytes_per_launch": ab,
                     "per_step_us": round(ms * 1e3, 3), "more_replays_us": extra_replays,
                     "launch_us_method": "eager launches" if args.eager_only else
                                         f"(median time of a {2 * args.steps}-launch graph - median time of the "
                                         f"{args.steps}-launch graph) / {args.steps}"},
        "us_per_call": round(ms * 1e3, 3),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "single_launch_us": single_launch(res, T),
    }
    extra = {}
    if args.eager_only:
        res.close()
        out["extra"] = extra
        print(json.dumps(out), flush=True)
        return

    # every decode line (all resident at once), interleaved rounds
    residents = {name: res}
    names = [] if args.primary_only else [n for n in qi.CONFIGS if n != name]
    if args.only:
        names = [n for n in names if n in args.only.split(",")]
    for n in names:
        residents[n] = Resident(n)
    lines = [(res, T2, 0) for T2 in qi.CONFIGS[name][3] if T2 != T]
    for n in names:
        lines += [(residents[n], T2, 0) for T2 in qi.CONFIGS[n][3]]
    # the explicit offset-operand route (QMAT_ROUTE_MFMA_OFFSET) on the Q4 gate+up matrix,
    # beside the automatic route's lines
    lines += [(res, T2, wq.QMAT_ROUTE_MFMA_OFFSET) for T2 in qi.CONFIGS[name][3]]
    results = measure_decode(lines, args.steps)
    for i, (r, T2, route) in enumerate(lines):
        key = f"{r.name}_T{T2}" + ("_offset_route" if route else "")
        extra[key] = results[i]
        log(f"[bench] {key}: {results[i]}")

    # the output-head epilogue on the Q6 head's logits (the last product left them in y)
    if "q6_head_248320x5120" in residents:
        r = residents["q6_head_248320x5120"]
        for T2 in qi.CONFIGS[r.name][3]:
            wq.qmat_run(r.handles[0], r.x[:T2], r.y[:T2], T=T2)
            key = f"head_epilogue_lse_top20_248320_T{T2}"
            extra[key] = measure_epilogue(r, T2, 20)
            log(f"[bench] {key}: {extra[key]}")
        for T2 in qi.CONFIGS[r.name][3]:
            key = f"head_product_and_epilogue_lse_top20_248320x5120_T{T2}"
            extra[key] = measure_epilogue(r, T2, 20, with_product=True)
            log(f"[bench] {key}: {extra[key]}")

    # prefill-sized token counts (the GEMM route)
    if not args.no_prefill:
        for n in [name] + [p for p in PREFILL_SHAPES if p in residents]:
            for T3 in PREFILL_T:
                key = f"{n}_prefill_T{T3}"
                extra[key] = measure_prefill(residents[n], T3, reference=(n == name))
                log(f"[bench] {key}: {extra[key]}")
    for r in residents.values():
        r.close()
    residents.clear()
    del res
    torch.cuda.empty_cache()

    if not args.no_ceiling:
        big = max(1 << 30, max(qmat_packed_size(n) for n in qi.CONFIGS) + (256 << 20)) // (1 << 20) * (1 << 20)
        c = read_ceilings(qmat_packed_size(name), big)
        out["read_stream_ceiling_GBps"] = c["GBps_big"]
        out["read_stream"] = c
        out["pct_of_read_ceiling"] = round(100 * value / c["GBps_big"], 2)
        out["pct_of_same_size_read"] = round(100 * value / c["GBps_window"], 2)
        out["same_size_read_us"] = round(c["window_bytes"] / (c["GBps_window"] * 1e3), 3)
        # every product line against the large read, and the matrices that rotate (< 512 MB)
        # also against a plain read of their own packed size (fixed launch, first-byte and drain
        # costs included), timed the same way
        windows = {name: c["GBps_window"]}
        for key, v in extra.items():
            if not ("GBps" in v and "bytes" in v and "k" not in v):
                continue
            v["pct_of_read_ceiling"] = round(100 * v["GBps"] / c["GBps_big"], 2)
            wname = key.rsplit("_T", 1)[0]
            size = qmat_packed_size(wname) // 1024 * 1024 if wname in qi.CONFIGS else 0
            if not 0 < size < (512 << 20):
                continue
            if wname not in windows:
                windows[wname], _ = read_probe_window(size)
            v["same_size_read_us"] = round(size / (windows[wname] * 1e3), 3)
            v["pct_of_same_size_read"] = round(100 * v["same_size_read_us"] / v["us_per_call"], 2)
        log(f"[bench] read stream: {c}")
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline ...")
        out["cpu_baseline"] = cpu_baseline(wl, T)
        log(f"[bench] cpu_baseline {out['cpu_baseline']}")
        out["cpu_context"] = cpu_context()
        log(f"[bench] cpu context {out['cpu_context']}")
    out["extra"] = extra
    print(json.dumps(out), flush=True)


def measured_traffic(workload):
    """HBM bytes per launch for a workload from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        from weight_only_quant_amd.rocprof_summary import kernel_source_sha256
        rec = json.load(open(path))
        if rec.get("kernel_source_sha256") != kernel_source_sha256():
            return None
        return int(round(rec["traffic_bytes"]))
    except Exception:
        return None


if __name__ == "__main__":
    main()
