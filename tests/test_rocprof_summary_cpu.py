"""The rocprofv3 summariser (measurement support) on small hand-made CSV files: durations, the
start-to-start period of back-to-back dispatches, per-dispatch counter means and the traffic
scaling by a copy of known size."""
import csv
import json

from weight_only_quant_amd import rocprof_summary as rs


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_durations_and_back_to_back_period(tmp_path):
    p = tmp_path / "kernel_trace.csv"
    H = ["Kernel_Name", "Grid_Size", "Workgroup_Size", "Start_Timestamp", "End_Timestamp"]
    k, o = "void qmatk::mfma_kernel<4, 2, 1>(qmatk::RunArgs)", "void other(int)"
    # three back-to-back launches of k (period 20 us), then another kernel, then k again
    rows = [[k, 100, 64, 0, 17000], [k, 100, 64, 20000, 37000], [k, 100, 64, 40000, 58000],
            [o, 8, 8, 60000, 61000], [k, 100, 64, 90000, 106000]]
    _write(p, H, rows[::-1])  # any order in the file
    out = {r["kernel"]: r for r in rs.trace_summary(str(p))}
    r = out["mfma_kernel<4, 2, 1>"]
    assert r["calls"] == 4 and r["grid"] == 100 and r["workgroup"] == 64
    assert abs(r["mean_us"] - (17 + 17 + 18 + 16) / 4) < 1e-9 and r["min_us"] == 16.0
    assert r["period_us"] == 20.0  # only the two back-to-back gaps count
    (other,) = [v for n, v in out.items() if "other" in n]
    assert other["calls"] == 1 and other["period_us"] is None


def test_counter_means_and_traffic(tmp_path):
    H = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    k = "void qmatk::mfma_kernel<4, 2, 1>(qmatk::RunArgs)"
    _write(tmp_path / "f.csv", H, [[k, 100, "FETCH_SIZE", 1000.0], [k, 100, "FETCH_SIZE", 3000.0],
                                   [k, 200, "FETCH_SIZE", 9.0]])
    _write(tmp_path / "w.csv", H, [[k, 100, "WRITE_SIZE", 10.0]])
    c = "__amd_rocclr_copyBuffer"
    _write(tmp_path / "cf.csv", H, [[c, 5, "FETCH_SIZE", 512.0]])   # a 1 MiB copy counted as half
    _write(tmp_path / "cw.csv", H, [[c, 5, "WRITE_SIZE", 1024.0]])  # ... and in full
    assert rs.counter_mean(str(tmp_path / "f.csv"), "FETCH_SIZE", "mfma_kernel", "100") == 2000.0
    out = tmp_path / "t.json"
    rs.main(["traffic", "--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
             "--copy-fetch", str(tmp_path / "cf.csv"), "--copy-write", str(tmp_path / "cw.csv"),
             "--copy-bytes", str(1 << 20), "--kernel", "mfma_kernel<4, 2, 1>", "--grid", "100",
             "--workload", "w", "--alg-bytes", "4096000", "--out", str(out)])
    rec = json.load(open(out))
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["traffic_bytes"] == 2000 * 1024 * 2 + 10 * 1024
