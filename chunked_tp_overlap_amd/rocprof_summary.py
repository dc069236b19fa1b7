"""Summarise rocprofv3 CSV output of ``bench.py --profile-pass ...`` into a short text report,
and (for the GEMMs) the HBM traffic figure that bench.py reports beside its roofline.

Three rocprofv3 runs of the same command feed it: a kernel trace with statistics, then one
counter pass for FETCH_SIZE and one for WRITE_SIZE.  Each profile pass ends with a plain
1 GiB device copy whose true traffic is known (2^30 bytes read, 2^30 written); each counter
is scaled by (known bytes / counted bytes) of that copy before it is applied to the
kernel's dispatches.

    python -m chunked_tp_overlap_amd.rocprof_summary --kt DIR --fetch DIR --write DIR \\
        --bench-json FILE [--key K] --kernel SUBSTRING --out profiles/x.md [--traffic FILE]

The profile pass's JSON line (or its sub-object --key) names the timed region:
timed_dispatches (the last that many dispatches whose name contains SUBSTRING, in every
run), timed_algorithmic_bytes, optionally timed_gflop, timed_calls and
hip_event_total_ms.  Everything is summed over those dispatches, so a sweep of shapes, or
calls that launch two kernels, is summarised as a whole: work over traced time, traffic
over algorithmic bytes.

--timeline DIR --bench-json FILE --out FILE instead summarises `bench.py --profile-pass
arrival` under `rocprofv3 --kernel-trace --memory-copy-trace`: per delivery mode, the
median call span, the time copies and GEMMs are active, and their overlap.

--streams DIR --bench-json FILE --out FILE summarises `bench.py --profile-pass host` under
`rocprofv3 --kernel-trace`: per mode, the median call span, the GEMM kernels' summed time,
the time at least one runs, their mean and maximum concurrency and the busy time per stream.

--util DIR adds a fourth run, --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES
SQ_BUSY_CU_CYCLES, read per dispatch with that run's own timestamps:
  - GRBM_GUI_ACTIVE sums the busy cycles of the 8 XCDs' GRBMs, so /8 is the dispatch's
    length in shader cycles, and over its duration the effective clock (an upper bound for
    short dispatches: the count includes the dispatch's set-up and drain);
  - SQ_VALU_MFMA_BUSY_CYCLES counts SIMD-cycles of issued MFMA work (1024 bf16 FLOP per
    SIMD-cycle), so against the algorithmic FLOPs it shows the MFMA work spent on the
    padded rows of partial tiles;
  - SQ_BUSY_CU_CYCLES sums the cycles each CU holds waves: over the dispatch's cycles, the
    mean number of busy CUs; against the MFMA cycles (4 SIMDs per CU), how busy the matrix
    cores of the busy CUs are.
"""

import argparse
import csv
import sys
import glob
import json
import os
import statistics

COPY_BYTES = 1 << 30


def _one(dirname, suffix):
    hits = glob.glob(os.path.join(dirname, f"*{suffix}"))
    if len(hits) != 1:
        raise SystemExit(f"expected one *{suffix} under {dirname}, found {hits}")
    return hits[0]


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def counter_sum(dirname, counter, kernel, n_timed):
    """Sum of `counter` (KiB) over the last n_timed dispatches of `kernel`, the number of
    them found, and the counter's value for the calibration copy."""
    rows = [r for r in _rows(_one(dirname, "_counter_collection.csv")) if r["Counter_Name"] == counter]
    by = {}
    for r in rows:
        if kernel in r["Kernel_Name"]:
            by[int(r["Dispatch_Id"])] = float(r["Counter_Value"])
    mine = [by[k] for k in sorted(by)][-n_timed:]
    # the calibration copy is the last and largest runtime copy of the pass (host-to-device
    # input uploads may show up as smaller copies before it)
    copy = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
    if not mine or not copy:
        raise SystemExit(f"{counter}: {len(mine)} dispatches of {kernel}, {len(copy)} copies")
    if copy[-1] != max(copy):
        raise SystemExit(f"{counter}: the last copy is not the largest: {copy}")
    return sum(mine), len(mine), copy[-1]


def counter_timed_dispatches(dirname, counters, kernel, n_timed):
    """Per-dispatch counter values (and duration in us, from the same run's timestamps) of
    the last n_timed dispatches of `kernel`."""
    by = {}
    for r in _rows(_one(dirname, "_counter_collection.csv")):
        if kernel not in r["Kernel_Name"] or r["Counter_Name"] not in counters:
            continue
        d = by.setdefault(int(r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    ds = [by[k] for k in sorted(by) if all(c in by[k] for c in counters)]
    if not ds:
        raise SystemExit(f"no dispatch of {kernel} with all of {counters}")
    return ds[-n_timed:]


UTIL_COUNTERS = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES")
LDS_COUNTERS = ("SQ_INSTS_LDS", "SQ_WAIT_INST_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS",
                "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_INSTS_MFMA")


def _union(iv):
    """Total length of the union of [start, end) intervals."""
    tot, cur_s, cur_e = 0, None, None
    for a, b in sorted(iv):
        if cur_e is None or a > cur_e:
            if cur_e is not None:
                tot += cur_e - cur_s
            cur_s, cur_e = a, b
        else:
            cur_e = max(cur_e, b)
    return tot + (cur_e - cur_s if cur_e is not None else 0)


def _intersect(xs, ys):
    """Length of (union of xs) intersected with (union of ys)."""
    return _union(xs) + _union(ys) - _union(list(xs) + list(ys))


def timeline(kt_dir, bench_json, out, title, command):
    """Per-call timelines of `bench.py --profile-pass arrival` from a kernel trace plus a
    memory-copy trace: the calls are the groups of events separated by the pass's 20 ms
    pauses that hold a GEMM; they are assigned to the pass's modes in order."""
    with open(bench_json) as f:
        top = json.loads([ln for ln in f if ln.startswith("{")][-1])
    ev = []
    for r in _rows(_one(kt_dir, "_kernel_trace.csv")):
        name = r["Kernel_Name"]
        kind = "gemm" if "gemm_bf16" in name else ("copy" if "copyBuffer" in name else "other")
        ev.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), kind, name[:48], r.get("Stream_Id", "")))
    for r in _rows(_one(kt_dir, "_memory_copy_trace.csv")):
        ev.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), "copy", r["Direction"], r.get("Stream_Id", "")))
    ev.sort()
    groups, cur, last_end = [], [], 0
    for e in ev:  # a gap of more than 5 ms after every event so far starts a new group
        if cur and e[0] - last_end > 5_000_000:
            groups.append(cur)
            cur = []
        if not cur:
            last_end = e[1]
        cur.append(e)
        last_end = max(last_end, e[1])
    if cur:
        groups.append(cur)
    calls = [g for g in groups if any(k == "gemm" for _, _, k, _, _ in g)]
    want = sum(m["calls"] for m in top["modes"])
    if len(calls) < want:
        raise SystemExit(f"found {len(calls)} calls with a GEMM, expected {want}")
    calls = calls[-want:]  # the pass's calls are the last ones
    lines = [f"# rocprofv3 summary: {title}", ""]
    if command:
        lines += ["Commands (from the repository root):", "", "```", command.strip(), "```", ""]
    lines += [f"T = {top['T']}, {top['chunks']} ring chunks, hardware queues {top.get('gpu_max_hw_queues')}, "
              f"wait timeouts {top.get('timeouts')}.  Per mode, medians over its calls (us):", "",
              "| mode | calls | call span | copies active | GEMMs active | both active | copies alone + GEMMs alone |",
              "|---|---|---|---|---|---|---|"]
    i = 0
    details = []
    for m in top["modes"]:
        rows = []
        for g in calls[i:i + m["calls"]]:
            t0 = g[0][0]
            cp = [(a, b) for a, b, k, _, _ in g if k == "copy"]
            gm = [(a, b) for a, b, k, _, _ in g if k == "gemm"]
            rows.append(((max(b for _, b, _, _, _ in g) - t0) / 1e3, _union(cp) / 1e3, _union(gm) / 1e3,
                         _intersect(cp, gm) / 1e3))
        i += m["calls"]
        med = [statistics.median(c[j] for c in rows) for j in range(4)]
        lines.append(f"| {m['mode']} | {m['calls']} | {med[0]:.1f} | {med[1]:.1f} | {med[2]:.1f} | {med[3]:.1f} | "
                     f"{med[1] + med[2]:.1f} |")
        g = calls[i - 1]
        t0 = g[0][0]
        details += ["", f"### {m['mode']}: its last call", "", "| kind | stream | start us | end us | name |",
                    "|---|---|---|---|---|"]
        details += [f"| {k} | {st} | {(a - t0) / 1e3:.1f} | {(b - t0) / 1e3:.1f} | `{n}` |" for a, b, k, n, st in g]
    lines += ["", "`both active` is the time during which a copy and a GEMM run at once (the overlap)."]
    lines += details
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines[:14 + len(top["modes"])]))


def _groups(ev, gap_ns=5_000_000):
    """Events (start, end, ...) sorted by start, split where a gap of more than gap_ns
    follows every event so far."""
    groups, cur, last_end = [], [], 0
    for e in ev:
        if cur and e[0] - last_end > gap_ns:
            groups.append(cur)
            cur = []
        if not cur:
            last_end = e[1]
        cur.append(e)
        last_end = max(last_end, e[1])
    if cur:
        groups.append(cur)
    return groups


def _max_concurrency(iv):
    pts = sorted([(a, 1) for a, _ in iv] + [(b, -1) for _, b in iv], key=lambda x: (x[0], x[1]))
    cur = best = 0
    for _, d in pts:
        cur += d
        best = max(best, cur)
    return best


def streams(kt_dir, bench_json, out, title, command):
    """Per-call stream timelines of `bench.py --profile-pass host` from a kernel trace: the
    calls are the groups of GEMM kernels separated by the pass's 20 ms pauses, assigned to
    the pass's modes in order.  Per call: span (first start to last end), the GEMM kernels'
    summed durations, the time at least one runs (union), their mean concurrency (sum /
    union), the most that run at once, the streams used, and the time each stream has a
    kernel running."""
    with open(bench_json) as f:
        top = json.loads([ln for ln in f if ln.startswith("{")][-1])
    ev = []
    for r in _rows(_one(kt_dir, "_kernel_trace.csv")):
        if "gemm_bf16" in r["Kernel_Name"]:
            ev.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r.get("Stream_Id", ""),
                       r["Kernel_Name"]))
    ev.sort()
    calls = _groups(ev)
    want = sum(m["calls"] for m in top["modes"])
    if len(calls) < want:
        raise SystemExit(f"found {len(calls)} calls, expected {want}")
    calls = calls[-want:]
    lines = [f"# rocprofv3 summary: {title}", ""]
    if command:
        lines += ["Commands (from the repository root):", "", "```", command.strip(), "```", ""]
    lines += [f"{top.get('workload')}: {top.get('chunks')} chunks on {top.get('streams')} streams "
              f"(host loop), hardware queues {top.get('gpu_max_hw_queues')}.  Per mode, medians over "
              f"its calls (the first call of each mode included):", "",
              "| mode | calls | span us | TFLOP/s over span | kernels | kernel sum us | union us | "
              "mean concurrency | max concurrency | streams | busy us per stream |",
              "|---|---|---|---|---|---|---|---|---|---|---|"]
    i = 0
    details = []
    for m in top["modes"]:
        rows = []
        for g in calls[i:i + m["calls"]]:
            iv = [(a, b) for a, b, _, _ in g]
            span = (max(b for _, b in iv) - g[0][0]) / 1e3
            ksum = sum(b - a for a, b in iv) / 1e3
            uni = _union(iv) / 1e3
            per = {}
            for a, b, st, _ in g:
                per.setdefault(st, []).append((a, b))
            busy = sorted((_union(v) / 1e3 for v in per.values()), reverse=True)
            rows.append((span, len(g), ksum, uni, ksum / uni, _max_concurrency(iv), len(per), busy))
        i += m["calls"]
        med = [statistics.median(r[j] for r in rows) for j in range(7)]
        busy = rows[len(rows) // 2][7]
        tf = m["gflop"] / med[0] * 1e3 if m.get("gflop") else 0.0  # GFLOP / us -> TFLOP/s
        lines.append(f"| {m['mode']} | {m['calls']} | {med[0]:.1f} | {tf:.0f} | {med[1]:.0f} | {med[2]:.1f} | "
                     f"{med[3]:.1f} | {med[4]:.2f} | {med[5]:.0f} | {med[6]:.0f} | "
                     f"{', '.join(f'{b:.1f}' for b in busy)} |")
        g = calls[i - 1]
        t0 = g[0][0]
        details += ["", f"### {m['mode']}: its last call", "", "| stream | start us | end us | us | kernel |",
                    "|---|---|---|---|---|"]
        details += [f"| {st} | {(a - t0) / 1e3:.1f} | {(b - t0) / 1e3:.1f} | {(b - a) / 1e3:.1f} | `{n[:60]}` |"
                    for a, b, st, n in g]
    lines += ["", "`mean concurrency` = summed kernel time / time at least one GEMM kernel runs."]
    lines += details
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines[:12 + len(top["modes"])]))


def main():
    if "--streams" in sys.argv:
        p = argparse.ArgumentParser()
        p.add_argument("--streams", required=True, help="rocprofv3 --kernel-trace directory")
        p.add_argument("--bench-json", required=True)
        p.add_argument("--title", default="host-loop stream timelines")
        p.add_argument("--command", default="")
        p.add_argument("--out", required=True)
        a = p.parse_args()
        streams(a.streams, a.bench_json, a.out, a.title, a.command)
        return
    if "--timeline" in sys.argv:
        p = argparse.ArgumentParser()
        p.add_argument("--timeline", required=True, help="rocprofv3 --kernel-trace --memory-copy-trace directory")
        p.add_argument("--bench-json", required=True)
        p.add_argument("--title", default="arrival stand-in timelines")
        p.add_argument("--command", default="")
        p.add_argument("--out", required=True)
        a = p.parse_args()
        timeline(a.timeline, a.bench_json, a.out, a.title, a.command)
        return
    p = argparse.ArgumentParser()
    p.add_argument("--kt", required=True, help="rocprofv3 --kernel-trace --stats output directory")
    p.add_argument("--fetch", required=True, help="rocprofv3 --pmc FETCH_SIZE output directory")
    p.add_argument("--write", required=True, help="rocprofv3 --pmc WRITE_SIZE output directory")
    p.add_argument("--bench-json", required=True, help="the JSON line the profiled command printed")
    p.add_argument("--key", default=None, help="sub-object of the JSON line for this kernel")
    p.add_argument("--kernel", required=True, help="substring of the kernel name")
    p.add_argument("--title", default=None)
    p.add_argument("--command", default="", help="the commands, for the report")
    p.add_argument("--out", required=True)
    p.add_argument("--traffic", default=None, help="write the traffic figure here (JSON)")
    p.add_argument("--util", default=None,
                   help="rocprofv3 --pmc " + " ".join(UTIL_COUNTERS) + " output directory")
    p.add_argument("--lds", default=None,
                   help="rocprofv3 --pmc " + " ".join(LDS_COUNTERS) + " output directory")
    p.add_argument("--peak-flop-per-cu-cycle", type=float, default=4096.0,
                   help="dense MFMA FLOP per CU per cycle of the kernel's dtype (bf16 4096, fp8 8192)")
    a = p.parse_args()

    with open(a.bench_json) as f:
        top = json.loads([ln for ln in f if ln.startswith("{")][-1])
    bench = top[a.key] if a.key else top
    n_timed = bench["timed_dispatches"]
    alg = bench["timed_algorithmic_bytes"]
    gflop = bench.get("timed_gflop")
    calls = bench.get("timed_calls", n_timed)

    stats = _rows(_one(a.kt, "_kernel_stats.csv"))
    trace = _rows(_one(a.kt, "_kernel_trace.csv"))
    mine = [r for r in trace if a.kernel in r["Kernel_Name"]]
    if len(mine) < n_timed:
        raise SystemExit(f"{len(mine)} dispatches of {a.kernel} in the trace, {n_timed} timed")
    timed = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in mine][-n_timed:]
    names = sorted({r["Kernel_Name"] for r in mine[-n_timed:]})
    t_total = sum(timed)  # us

    f_sum, f_n, f_copy = counter_sum(a.fetch, "FETCH_SIZE", a.kernel, n_timed)
    w_sum, w_n, w_copy = counter_sum(a.write, "WRITE_SIZE", a.kernel, n_timed)
    f_scale = (COPY_BYTES / 1024) / f_copy
    w_scale = (COPY_BYTES / 1024) / w_copy
    traffic_total = f_sum * 1024 * f_scale + w_sum * 1024 * w_scale

    lines = [f"# rocprofv3 summary: {a.title or a.kernel}", ""]
    if a.command:
        lines += ["Commands (from the repository root):", "", "```", a.command.strip(), "```", ""]
    lines += ["## Kernel trace (--kernel-trace --stats)", "",
              "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{r['Name'][:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    lines += ["", "Timed region: the last "
              f"{n_timed} dispatches whose name contains `{a.kernel}` ({calls} library calls); "
              f"kernels among them:", ""]
    lines += [f"- `{n[:150]}`" for n in names]
    lines += ["",
              f"- traced kernel time: {t_total / 1e3:.3f} ms in total, {t_total / n_timed:.2f} us per "
              f"dispatch, {t_total / calls:.2f} us per call"]
    if bench.get("hip_event_total_ms"):
        ev = bench["hip_event_total_ms"] * 1e3
        lines.append(f"- the profiled command's own per-call HIP events: {ev / 1e3:.3f} ms in total "
                     f"(trace / events = {t_total / ev:.3f})")
    lines.append(f"- algorithmic bytes: {alg / 1e6:.2f} MB, i.e. {alg / t_total / 1e3:.1f} GB/s over "
                 f"the traced time")
    if gflop:
        lines.append(f"- algorithmic work: {gflop:.3f} GFLOP, i.e. {gflop / t_total * 1e3:.1f} TFLOP/s "
                     f"over the traced time")
    lines += ["", "## HBM-side traffic (--pmc FETCH_SIZE, then --pmc WRITE_SIZE)", "",
              "| counter | timed dispatches | kernel KiB (raw, summed) | 1 GiB copy (raw KiB) | scale | "
              "kernel MB (scaled) |", "|---|---|---|---|---|---|",
              f"| FETCH_SIZE | {f_n} | {f_sum:.1f} | {f_copy:.1f} | {f_scale:.4f} | "
              f"{f_sum * 1024 * f_scale / 1e6:.2f} |",
              f"| WRITE_SIZE | {w_n} | {w_sum:.1f} | {w_copy:.1f} | {w_scale:.4f} | "
              f"{w_sum * 1024 * w_scale / 1e6:.2f} |", "",
              f"Scaled traffic: {traffic_total / 1e6:.2f} MB over the timed region "
              f"({traffic_total / calls / 1e6:.2f} MB per call), against {alg / 1e6:.2f} MB "
              f"algorithmic ({traffic_total / alg:.2f}x).", "",
              f"Kernel source: {top['src_file']}, sha256[:16] {top['src_hash']}"]
    util = None
    if a.util:
        ds = counter_timed_dispatches(a.util, UTIL_COUNTERS, a.kernel, n_timed)
        tot = {c: sum(d[c] for d in ds) for c in UTIL_COUNTERS + ("us",)}
        cyc = tot["GRBM_GUI_ACTIVE"] / 8               # shader cycles of the dispatches
        mfma, cu_busy = tot["SQ_VALU_MFMA_BUSY_CYCLES"], tot["SQ_BUSY_CU_CYCLES"]
        mhz = cyc / tot["us"]
        util = {"effective_clock_mhz": round(mhz, 1),
                "peak_at_clock_tflops": round(256 * a.peak_flop_per_cu_cycle * mhz / 1e6, 1),
                "busy_cus_mean": round(cu_busy / cyc, 1),
                "mfma_active_of_busy_cu_cycles": round(mfma / (4 * cu_busy), 4),
                "mfma_active_of_all_cu_cycles": round(mfma / (4 * 256 * cyc), 4)}
        if gflop:
            need = gflop * 1e9 / (a.peak_flop_per_cu_cycle / 4)  # SIMD-cycles
            util["mfma_issued_per_algorithmic"] = round(mfma / need, 4)
        lines += ["", "## Clock and MFMA activity (--pmc " + " ".join(UTIL_COUNTERS) + ")", "",
                  f"Sums over the last {len(ds)} dispatches of the counter run (its own timestamps: "
                  f"{tot['us'] / 1e3:.3f} ms of kernel time):", "",
                  "| counter | total |", "|---|---|"]
        lines += [f"| {c} | {tot[c]:.5g} |" for c in UTIL_COUNTERS]
        lines += ["",
                  f"- length: GRBM_GUI_ACTIVE / 8 XCDs = {cyc:.4g} cycles; over "
                  f"{tot['us'] / 1e3:.3f} ms, an effective clock of {mhz:.0f} MHz (nominal 2400; an "
                  f"upper bound, the count includes each dispatch's set-up and drain)",
                  f"- busy CUs: SQ_BUSY_CU_CYCLES / cycles = {cu_busy / cyc:.1f} of 256 on average",
                  f"- matrix cores of the busy CUs: MFMA SIMD-cycles / (4 x busy CU-cycles) = "
                  f"{mfma / (4 * cu_busy):.3f}",
                  f"- matrix cores of the whole chip: {mfma / (4 * 256 * cyc):.3f}"]
        if gflop:
            lines.append(f"- MFMA work issued: {mfma:.4g} SIMD-cycles, {util['mfma_issued_per_algorithmic']:.3f}x "
                         f"the algorithmic FLOPs at {a.peak_flop_per_cu_cycle / 4:.0f} FLOP per "
                         f"SIMD-cycle (the excess is padded rows of partial tiles)")
    if a.lds:
        ds = counter_timed_dispatches(a.lds, LDS_COUNTERS, a.kernel, n_timed)
        tot = {c: sum(d[c] for d in ds) for c in LDS_COUNTERS}
        ratio = lambda x, y: tot[x] / tot[y] if tot[y] else float("nan")
        lines += ["", "## Where the waves wait (--pmc " + " ".join(LDS_COUNTERS) + ")", "",
                  f"Sums over the last {len(ds)} dispatches of the counter run:", "",
                  "| counter | total |", "|---|---|"]
        lines += [f"| {c} | {tot[c]:.5g} |" for c in LDS_COUNTERS]
        lines += ["",
                  f"- LDS instructions per MFMA instruction: SQ_INSTS_LDS / SQ_INSTS_MFMA = "
                  f"{ratio('SQ_INSTS_LDS', 'SQ_INSTS_MFMA'):.3f}",
                  f"- bank conflicts: SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS = "
                  f"{ratio('SQ_LDS_BANK_CONFLICT', 'SQ_ACTIVE_INST_LDS'):.4f} of the LDS-active cycles",
                  f"- wave-cycles spent waiting to issue an LDS instruction: SQ_WAIT_INST_LDS / "
                  f"SQ_WAVE_CYCLES = {ratio('SQ_WAIT_INST_LDS', 'SQ_WAVE_CYCLES'):.4f}",
                  f"- wave-cycles spent waiting on any dependency or counter: SQ_WAIT_ANY / "
                  f"SQ_WAVE_CYCLES = {ratio('SQ_WAIT_ANY', 'SQ_WAVE_CYCLES'):.4f}"]
        if gflop:
            lines.append(f"- MFMA math issued: SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 FLOP = "
                         f"{tot['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / 1e9:.1f} GFLOP against "
                         f"{gflop:.1f} algorithmic ({tot['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / 1e9 / gflop:.3f}x)")
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    if a.traffic:
        with open(a.traffic, "w") as f:
            json.dump({"workload": top.get("profile_pass"), "src_file": top["src_file"],
                       "src_hash": top["src_hash"], "kernel": a.kernel,
                       "source": os.path.relpath(a.out),
                       "bytes_per_call": round(traffic_total / calls),
                       "algorithmic_bytes_per_call": round(alg / calls),
                       "traffic_over_algorithmic": round(traffic_total / alg, 4),
                       "fetch_kib_raw_total": round(f_sum, 2), "fetch_scale": round(f_scale, 5),
                       "write_kib_raw_total": round(w_sum, 2), "write_scale": round(w_scale, 5),
                       "trace_us_per_call": round(t_total / calls, 3), "util": util}, f, indent=1)
            f.write("\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
