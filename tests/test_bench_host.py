"""Host-side checks of the benchmark harness: the one-GPU guard, the rocprofv3 summariser's
arithmetic on synthetic CSVs, and the device-state record's failure path (no GPU here)."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL = "void ubx::gemm_bf16_pingpong<Cfg<256, 256>>(Params)"


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr
    assert r.stdout.strip() == ""


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _counter_dir(base, name, values, copy_kib=None):
    """A rocprofv3-like counter CSV: `values` = list of {counter: value} per kernel
    dispatch (100 us each), then optionally one calibration copy."""
    d = base / name
    d.mkdir()
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    rows, t = [], 1_000_000
    for i, v in enumerate(values):
        for c, x in v.items():
            rows.append([i, KERNEL, c, x, t, t + 100_000])
        t += 200_000
    if copy_kib is not None:
        for c, x in copy_kib.items():
            rows.append([len(values), "__amd_rocclr_copyBuffer", c, x, t, t + 1000])
    _write(d / f"{name}_counter_collection.csv", hdr, rows)
    return d


@pytest.fixture()
def profile_dirs(tmp_path):
    kt = tmp_path / "kt"
    kt.mkdir()
    _write(kt / "kt_kernel_stats.csv", ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
           [[KERNEL, 4, 100000, 90000, 110000]])
    # 4 dispatches: the first 2 untimed (300 us), the last 2 timed (100 us)
    _write(kt / "kt_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           [[KERNEL, 0, 300_000], [KERNEL, 0, 300_000], [KERNEL, 0, 100_000], [KERNEL, 0, 100_000]])
    # raw FETCH counts half the copy's true 1 GiB read, WRITE counts it exactly
    fetch = _counter_dir(tmp_path, "fetch", [{"FETCH_SIZE": 1000.0}] * 4,
                         {"FETCH_SIZE": (1 << 30) / 1024 / 2})
    write = _counter_dir(tmp_path, "write", [{"WRITE_SIZE": 500.0}] * 4,
                         {"WRITE_SIZE": (1 << 30) / 1024})
    # 2.4e5 GUI cycles summed over 8 XCDs in 100 us -> 300 MHz; MFMA and CU-busy counts
    util = _counter_dir(tmp_path, "util", [{"GRBM_GUI_ACTIVE": 240000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 2.0e6,
                                            "SQ_BUSY_CU_CYCLES": 3.0e6}] * 4)
    bench = tmp_path / "b.json"
    bench.write_text("[bench] log line\n" + json.dumps({
        "profile_pass": "gqa", "timed_dispatches": 2, "timed_calls": 1, "hip_event_total_ms": 0.21,
        "timed_gflop": 4.096, "timed_algorithmic_bytes": 2_000_000, "src_file": "x.hip",
        "src_hash": "abc"}) + "\n")
    return kt, fetch, write, util, bench


def test_rocprof_summary_arithmetic(profile_dirs, tmp_path):
    kt, fetch, write, util, bench = profile_dirs
    out, traffic = tmp_path / "s.md", tmp_path / "t.json"
    r = subprocess.run([sys.executable, "-m", "chunked_tp_overlap_amd.rocprof_summary", "--kt", str(kt),
                        "--fetch", str(fetch), "--write", str(write), "--util", str(util),
                        "--bench-json", str(bench), "--kernel", "gemm_bf16_pingpong",
                        "--out", str(out), "--traffic", str(traffic)],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    t = json.loads(traffic.read_text())
    # the last 2 dispatches are timed, making 1 call: fetch scaled x2 (the copy read half of
    # 1 GiB), write x1, summed over the 2 dispatches: 2 * (1000*2 + 500) KiB per call
    assert t["fetch_scale"] == pytest.approx(2.0)
    assert t["write_scale"] == pytest.approx(1.0)
    assert t["bytes_per_call"] == 2 * (1000 * 2 + 500) * 1024
    assert t["algorithmic_bytes_per_call"] == 2_000_000
    assert t["trace_us_per_call"] == pytest.approx(200.0)   # the timed (last 2) dispatches only
    assert t["workload"] == "gqa" and t["src_hash"] == "abc"
    u = t["util"]
    cyc = 2 * 240000.0 / 8                                   # 6e4 cycles over 200 us
    assert u["effective_clock_mhz"] == pytest.approx(cyc / 200.0)
    assert u["busy_cus_mean"] == pytest.approx(2 * 3.0e6 / cyc, abs=0.05)
    assert u["mfma_active_of_busy_cu_cycles"] == pytest.approx(2.0e6 / (4 * 3.0e6), abs=1e-4)
    assert u["mfma_active_of_all_cu_cycles"] == pytest.approx(2 * 2.0e6 / (4 * 256 * cyc), abs=1e-4)
    # 4.096 GFLOP at 1024 FLOP per SIMD-cycle = 4e6 SIMD-cycles: issued == algorithmic
    assert u["mfma_issued_per_algorithmic"] == pytest.approx(1.0, abs=1e-4)
    md = out.read_text()
    assert "(2.56x)" in md                   # 5.12 MB scaled against 2.00 MB
    assert "20.5 TFLOP/s" in md              # 4.096 GFLOP over 200 us


def test_rocprof_summary_rejects_out_of_order_copies(profile_dirs, tmp_path):
    kt, _, write, _, bench = profile_dirs
    bad = _counter_dir(tmp_path, "badfetch", [{"FETCH_SIZE": 1000.0}] * 4)
    with open(bad / "badfetch_counter_collection.csv", "a", newline="") as f:
        w = csv.writer(f)
        w.writerow([9, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 999999.0, 0, 1])
        w.writerow([10, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 10.0, 0, 1])
    r = subprocess.run([sys.executable, "-m", "chunked_tp_overlap_amd.rocprof_summary", "--kt", str(kt),
                        "--fetch", str(bad), "--write", str(write), "--bench-json", str(bench),
                        "--kernel", "gemm_bf16_pingpong", "--out", str(tmp_path / "s.md")],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "not the largest" in (r.stderr + r.stdout)


def test_device_state_fails_softly_without_gpu():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("host-only check")
    sys.path.insert(0, ROOT)
    import bench

    s = bench.device_state(torch)
    assert s["power_cap_w"] is None and s["error"]


def test_timeline_summary_on_synthetic_trace(tmp_path):
    """Two modes, two calls each, 20 ms apart: copies [0, 100) and [100, 200) us with GEMMs
    [50, 150) and [150, 250) us in every call of mode a; mode b has no overlap."""
    d = tmp_path / "tr"
    d.mkdir()
    kt, mc = [], []
    t = 50_000_000
    for mode in ("a", "b"):
        for _ in range(2):
            if mode == "a":
                mc += [["MEMORY_COPY_HOST_TO_DEVICE", t, t + 100_000, 3], ["MEMORY_COPY_HOST_TO_DEVICE", t + 100_000, t + 200_000, 3]]
                kt += [[KERNEL, t + 50_000, t + 150_000, 0], [KERNEL, t + 150_000, t + 250_000, 1]]
            else:
                mc += [["MEMORY_COPY_DEVICE_TO_DEVICE", t, t + 100_000, 3]]
                kt += [[KERNEL, t + 100_000, t + 180_000, 0]]
            t += 20_000_000
    kt.insert(0, ["void at::native::fill(int)", 1_000_000, 1_010_000, 0])  # setup, no GEMM
    _write(d / "tr_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Stream_Id"], kt)
    _write(d / "tr_memory_copy_trace.csv", ["Direction", "Start_Timestamp", "End_Timestamp", "Stream_Id"], mc)
    bench = tmp_path / "b.json"
    bench.write_text(json.dumps({"profile_pass": "arrival", "T": 8192, "chunks": 8, "timeouts": 0,
                                 "modes": [{"mode": "a", "calls": 2}, {"mode": "b", "calls": 2}]}) + "\n")
    out = tmp_path / "tl.md"
    r = subprocess.run([sys.executable, "-m", "chunked_tp_overlap_amd.rocprof_summary", "--timeline", str(d),
                        "--bench-json", str(bench), "--out", str(out)],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    md = out.read_text()
    assert "| a | 2 | 250.0 | 200.0 | 200.0 | 150.0 | 400.0 |" in md
    assert "| b | 2 | 180.0 | 100.0 | 80.0 | 0.0 | 180.0 |" in md


def test_call_dispatches_and_plan_text():
    """Dispatch count of a call from its plan: plain rows once (twice when cut), split-K
    rows once when summed in the kernel or folded, twice with the separate sum."""
    import bench
    plain = (1024, 256, 256, -1, 0, 0, -1, 0, 0, 0, 0)
    cut = (1024, 320, 256, 6400, 128, 128, -1, 0, 0, 0, 0)
    seg_only = (1024, 128, 256, -1, 0, 0, 0, 6, 2, 128, 256)
    lead_seg = (13216, 320, 256, -1, 0, 0, 13056, 12, 2, 128, 128)
    lead_cut_seg = (13216, 320, 256, 6400, 256, 256, 13056, 4, 1, 256, 256)
    folded = (1024, 128, 128, -1, 0, 0, 0, 6, 0, 128, 128)
    assert [bench._call_dispatches(p) for p in (plain, cut, seg_only, lead_seg, lead_cut_seg, folded)] == \
        [1, 2, 2, 3, 3, 1]
    assert bench.describe_plan(plain[1:]) == "256x256"
    assert bench.describe_plan(cut[1:]) == "320x256 cut 6400: 128x128"
    assert bench.describe_plan(seg_only[1:]) == "split-K from row 0: 6 x 128x256 r2"
    assert bench.describe_plan(lead_seg[1:]) == "320x256; split-K from row 13056: 12 x 128x128 r2"
    assert bench.describe_plan(folded[1:]) == "split-K from row 0: 6 x 128x128 fold"


def test_streams_summary_on_synthetic_trace(tmp_path):
    """Host-loop timelines: mode a runs three kernels on three streams, two of them at once
    ([0, 100), [50, 150), [150, 200) us); mode b two kernels back to back on one stream."""
    d = tmp_path / "kt"
    d.mkdir()
    kt = []
    t = 50_000_000
    for mode in ("a", "b"):
        for _ in range(2):
            if mode == "a":
                kt += [[KERNEL, t, t + 100_000, 1], [KERNEL, t + 50_000, t + 150_000, 2],
                       [KERNEL, t + 150_000, t + 200_000, 3]]
            else:
                kt += [[KERNEL, t, t + 60_000, 0], [KERNEL, t + 60_000, t + 100_000, 0]]
            t += 20_000_000
    kt.insert(0, ["void at::native::fill(int)", 1_000_000, 1_010_000, 0])
    _write(d / "kt_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Stream_Id"], kt)
    bench = tmp_path / "b.json"
    bench.write_text(json.dumps({"profile_pass": "host", "workload": "w", "chunks": 8, "streams": 3,
                                 "modes": [{"mode": "a", "calls": 2, "gflop": 20.0},
                                           {"mode": "b", "calls": 2, "gflop": 10.0}]}) + "\n")
    out = tmp_path / "st.md"
    r = subprocess.run([sys.executable, "-m", "chunked_tp_overlap_amd.rocprof_summary", "--streams", str(d),
                        "--bench-json", str(bench), "--out", str(out)],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    md = out.read_text()
    # span 200 us, 20 GFLOP -> 100 TFLOP/s; sum 250, union 200, mean 1.25, max 2, 3 streams
    assert "| a | 2 | 200.0 | 100 | 3 | 250.0 | 200.0 | 1.25 | 2 | 3 | 100.0, 100.0, 50.0 |" in md
    assert "| b | 2 | 100.0 | 100 | 2 | 100.0 | 100.0 | 1.00 | 1 | 1 | 100.0 |" in md
