"""Benchmark of the weight-only quantized small-T product on one MI355X.

A step is one qmat_run call (the whole product: stream packed codes and scales, unpack,
dot products, group scales, reductions, write y) on resident device buffers.  The headline
workload is the Q4 fused MLP gate+up projection (two 17408 x 5120 matrices as one
M=34816, K=5120 matrix) at T=1; the other benchmark shapes (Q6 vocab head, Q5 down
projection with split-K, FP8 row-scaled head and projection, the small Q4 case) at each
of their token counts are reported in "extra".

Throughput is algorithmic bytes (packed codes + scales read once, x read, y written) per
second.  Matrices smaller than 512 MB rotate over enough device copies to exceed 512 MB so
the 256 MB Infinity Cache cannot serve them.  Inputs are seeded synthetic data.

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
PREFILL_SHAPES = ("q5_down_5120x17408", "fp8_proj_5120x5120")


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


def time_run(res, T, steps, warmup):
    """Eager stream launches.  Returns (ms_per_step over the timed region, and the per-launch
    kernel ms from HIP events bracketing each launch on the launch stream: mean, median, 10th
    and 90th percentiles)."""
    import torch
    import weight_only_quant_amd as wq
    stream = torch.cuda.current_stream()
    x, y = res.x[:T], res.y[:T]
    hs = res.handles
    for i in range(warmup):
        wq.qmat_run(hs[i % len(hs)], x, y, T=T, stream=stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        ev[i][0].record(stream)
        wq.qmat_run(hs[i % len(hs)], x, y, T=T, stream=stream)
        ev[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    total = start.elapsed_time(end)
    per = [a.elapsed_time(b) for a, b in ev]
    return (total / steps, float(np.mean(per)), float(np.median(per)), float(np.percentile(per, 10)),
            float(np.percentile(per, 90)))


def time_graph(res, T, steps, warmup):
    """The same K steps captured once into a HIP graph and replayed: the way a decode step
    is launched in an engine.  Returns ms per step over the timed replay."""
    import gc
    import torch
    import weight_only_quant_amd as wq
    x, y = res.x[:T], res.y[:T]
    hs = res.handles
    gc.collect()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            wq.qmat_run(hs[i % len(hs)], x, y, T=T)
    for _ in range(max(1, warmup // steps)):
        g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    del g
    return ms


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


def qmat_packed_size(name):
    """Packed bytes (codes + scales) of a benchmark workload."""
    import qmat_inputs as qi
    import weight_only_quant_amd as wq
    c = qi.CONFIGS[name]
    return wq.qmat_packed_bytes(c[0], c[1], c[2])


def plan_str(res, T):
    import weight_only_quant_amd as wq
    p = wq.qmat_get_plan(res.handles[0], T)
    tail = f" tail_tiles={p.tail_tiles} tail_splits={p.tail_splits}" if p.tail_tiles else ""
    tiles = f" tiles={p.tiles}" if p.tiles > 1 else ""
    return (f"{'valu' if p.route == wq.QMAT_ROUTE_VALU else 'mfma'} depth={p.depth} waves={p.waves} "
            f"splits={p.splits}{tail}{tiles}")


EAGER_ONLY = False


def measure(res, T, steps, warmup):
    ms_e, k_mean, k_med, k_p10, k_p90 = time_run(res, T, steps, warmup)
    ms_g = ms_e if EAGER_ONLY else time_graph(res, T, steps, warmup)
    wl = res.wl
    ab = alg_bytes(wl.fmt, wl.M, wl.K, T)
    return {"us_per_call": round(ms_g * 1e3, 3), "eager_us_per_call": round(ms_e * 1e3, 3),
            "kernel_us": round(k_mean * 1e3, 3), "kernel_us_median": round(k_med * 1e3, 3),
            "kernel_us_p10": round(k_p10 * 1e3, 3), "kernel_us_p90": round(k_p90 * 1e3, 3),
            "GBps": round(ab / (ms_g * 1e-3) / 1e9, 1), "kernel_GBps": round(ab / (k_mean * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * ab / (ms_g * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "bytes": ab, "plan": plan_str(res, T)}


def measure_epilogue(res, T, k, steps, warmup):
    """The output-head epilogue (per-token log-sum-exp and top-k) on the logits the head product
    left in res.y, graph-replayed; bytes are the logits read (T * M * 4)."""
    import torch
    import weight_only_quant_amd as wq
    M = res.wl.M
    e = wq.qmat_logits_create(M, T, k)
    y = res.y[:T]
    lse = torch.empty(T, device="cuda")
    v = torch.empty((T, k), device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    for _ in range(warmup):
        wq.qmat_logits_run(e, y, k, lse=lse, top_vals=v, top_ids=ids)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            wq.qmat_logits_run(e, y, k, lse=lse, top_vals=v, top_ids=ids)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / steps * 1e3
    del g
    wq.qmat_logits_destroy(e)
    nb = T * M * 4
    return {"us_per_call": round(us, 3), "GBps": round(nb / us / 1e3, 1), "bytes": nb, "k": k}


def measure_prefill(res, T, steps=20, warmup=3, reference=False):
    """A prefill-sized product (the GEMM route) on the resident matrix with T synthetic bf16
    activation rows; throughput in TFLOP/s (2 T M K per call)."""
    import torch
    import weight_only_quant_amd as wq
    wl = res.wl
    g = torch.Generator(device="cuda")
    g.manual_seed(T)
    x = torch.randn((T, wl.K), generator=g, device="cuda").to(torch.bfloat16)
    y = torch.empty((T, wl.M), device="cuda")
    hs = res.handles
    for i in range(warmup):
        wq.qmat_run(hs[i % len(hs)], x, y, T=T)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        wq.qmat_run(hs[i % len(hs)], x, y, T=T)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / steps * 1e3
    tf = 2.0 * T * wl.M * wl.K / us / 1e6
    out = {"us_per_call": round(us, 2), "TFLOPs": round(tf, 1), "pct_bf16_mfma_peak": round(100 * tf / 2500.0, 2),
           "route": "gemm"}
    if reference:
        # context, not the product: the vendor bf16 GEMM (torch.matmul -> hipBLASLt) on an
        # unquantized bf16 weight of the same shape, the practical matrix-core rate on this GPU
        w = torch.randn((wl.M, wl.K), generator=g, device="cuda").to(torch.bfloat16)
        for i in range(warmup):
            torch.matmul(x, w.t())
        torch.cuda.synchronize()
        a.record()
        for i in range(steps):
            torch.matmul(x, w.t())
        b.record()
        torch.cuda.synchronize()
        ref_us = a.elapsed_time(b) / steps * 1e3
        out["bf16_vendor_gemm_us"] = round(ref_us, 2)
        out["bf16_vendor_gemm_TFLOPs"] = round(2.0 * T * wl.M * wl.K / ref_us / 1e6, 1)
        del w
    del x, y
    return out


def cpu_baseline(res, T, target_s=12.0):
    """The CPU oracle (as it stands) on a bounded sample of the same workload: whole passes
    over all rows (or a row subset when one pass would exceed the budget), repeated until
    about target_s seconds of CPU work have run."""
    import oracle
    wl = res.wl
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


def read_ceilings(window_bytes):
    """Practical read-bandwidth ceilings from the read-stream probe (libqmat_probe.so, a plain
    16-byte-per-lane nontemporal read; best of a few launch shapes): over a 1 GiB buffer, and
    over windows of the headline matrix's size rotated through that buffer (so each read
    streams from HBM, as the rotated weight copies do)."""
    from weight_only_quant_amd import probe
    big, big_shapes = probe.best_read_gbs(1 << 30)
    w = window_bytes // 1024 * 1024
    win, _ = probe.best_read_gbs(1 << 30, window=w, reps=100)
    return {"GBps_1GiB": big, "shapes_1GiB": big_shapes, "GBps_window": win, "window_bytes": w}


def read_probe_window(window_bytes):
    """Best plain-read rate (GB/s) over windows of window_bytes rotated through 1 GiB."""
    from weight_only_quant_amd import probe
    return probe.best_read_gbs(1 << 30, window=window_bytes, reps=100)


def cpu_context(target_s=1.0):
    """The host CPU model and the oracle's single-thread time on the small Q4 case (256 x 1024,
    T = 1), the one the measurement plan times on one core."""
    import oracle
    import qmat_inputs as qi
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
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
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=800)
    ap.add_argument("--primary-only", action="store_true", help="skip the other benchmark shapes")
    ap.add_argument("--only", default=None, help="comma-separated config names for the extra shapes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 256 MiB device copy (known bytes) for scaling PMC byte counters")
    ap.add_argument("--eager-only", action="store_true",
                    help="time eager stream launches only (no graph replay), e.g. under a counter profiler")
    args = ap.parse_args()
    global EAGER_ONLY
    EAGER_ONLY = args.eager_only
    if args.gpus != 1:
        log("bench.py: the benchmark runs on one GPU only (the product shards by rows with no "
            "collective; see the design notes); --gpus must be 1")
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

    name, T = PRIMARY
    res = Resident(name)
    wl = res.wl
    m = measure(res, T, args.steps, args.warmup)
    ab = m["bytes"]
    ms = m["us_per_call"] * 1e-3
    value = ab / (ms * 1e-3) / 1e9
    # one launch per step: the average launch duration is the graph-replay time per step
    # (kernel plus the inter-kernel gap); per-launch event brackets add their own flushes
    achieved = value
    log(f"[bench] {name} T={T}: {m}")
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
                   "launch": "eager stream launches" if EAGER_ONLY else "K steps captured in one HIP graph and replayed",
                   "plan": m["plan"]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(f"{name}_T{T}"),
                     "launch_us_mean": m["us_per_call"], "event_bracketed_launch_us_mean": m["kernel_us"],
                     "event_bracketed_launch_us_median": m["kernel_us_median"], "bytes_per_launch": ab},
        "us_per_call": m["us_per_call"],
        "eager_us_per_call": m["eager_us_per_call"],
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
    }
    extra = {}
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline ...")
        out["cpu_baseline"] = cpu_baseline(res, T)
        log(f"[bench] cpu_baseline {out['cpu_baseline']}")
    # the same workload at its other token counts
    for T2 in qi.CONFIGS[name][3]:
        if T2 == T:
            continue
        extra[f"{name}_T{T2}"] = measure(res, T2, args.steps, args.warmup)
        log(f"[bench] {name} T={T2}: {extra[f'{name}_T{T2}']}")
    # prefill-sized token counts (the GEMM route)
    for T2 in PREFILL_T:
        key = f"{name}_prefill_T{T2}"
        extra[key] = measure_prefill(res, T2, reference=True)
        log(f"[bench] {key}: {extra[key]}")
    res.close()
    del res
    torch.cuda.empty_cache()
    if not args.primary_only:
        names = [n for n in qi.CONFIGS if n != name]
        if args.only:
            names = [n for n in names if n in args.only.split(",")]
        for n in names:
            r = Resident(n)
            for T2 in qi.CONFIGS[n][3]:
                steps = args.steps if r.wl.M * r.wl.K < 1e9 else max(50, args.steps // 4)
                extra[f"{n}_T{T2}"] = measure(r, T2, steps, args.warmup)
                log(f"[bench] {n} T={T2}: {extra[f'{n}_T{T2}']}")
                if n in PREFILL_SHAPES and T2 == qi.CONFIGS[n][3][0]:
                    for T3 in PREFILL_T:
                        key = f"{n}_prefill_T{T3}"
                        extra[key] = measure_prefill(r, T3)
                        log(f"[bench] {key}: {extra[key]}")
                if n == "q6_head_248320x5120":
                    key = f"head_epilogue_lse_top20_248320_T{T2}"
                    extra[key] = measure_epilogue(r, T2, 20, args.steps, 20)
                    log(f"[bench] {key}: {extra[key]}")
            r.close()
            del r
            torch.cuda.empty_cache()
    if not args.no_ceiling:
        c = read_ceilings(qmat_packed_size(name))
        out["read_stream_ceiling_GBps"] = c["GBps_1GiB"]
        out["read_stream"] = c
        out["pct_of_read_ceiling"] = round(100 * value / c["GBps_1GiB"], 2)
        out["pct_of_same_size_read"] = round(100 * value / c["GBps_window"], 2)
        out["same_size_read_us"] = round(c["window_bytes"] / (c["GBps_window"] * 1e3), 3)
        # every product line against the 1 GiB read, and the matrices that rotate (< 512 MB)
        # also against a plain read of their own packed size (fixed launch, first-byte and drain
        # costs included), timed the same way
        windows = {name: c["GBps_window"]}
        for key, v in extra.items():
            if not ("GBps" in v and "bytes" in v and "k" not in v):
                continue
            v["pct_of_read_ceiling"] = round(100 * v["GBps"] / c["GBps_1GiB"], 2)
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
        out["cpu_context"] = cpu_context()
        log(f"[bench] cpu context {out['cpu_context']}")
    out["extra"] = extra
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
