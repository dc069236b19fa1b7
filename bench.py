#!/usr/bin/env python3
"""Benchmark of the chunked tensor-parallel overlap GEMMs on one MI355X.

Metric: bf16 TFLOP/s of the chunked AG/RS GEMM at the active T, and its fraction of the
dense bf16 MFMA peak.  The headline workload is the largest single-GPU configuration, the
GQA QKV all-gather-side GEMM in bulk mode: one UserBuffer registered once at capacity
[32768, 8192], W [8192, 1280], tp 8, num_splits 8, and a T sweep from 1024 to 32520 in steps
of 1016 (32 points) on that one registration, with no reallocation between points.  One
step = the whole sweep: for each T, ub_set_active_shape([T, 8192]) then one
ub_gemm_ag_chunked call.  FLOPs are algorithmic: 2 * T * 8192 * 1280 per point, active T
only.  Inputs are seeded synthetic draws already resident in HBM when the timed region
starts.

The schedule is the device-side chunk loop (option atomic_gemm: one launch per call, or two
when the plan cuts a nearly empty last round, whose workgroups walk the 8 chunks in plan
order); the host loop of per-chunk launches on min(8, 3) streams is measured as a secondary
row, as are the QKV, fc1 and fc2 workloads, the reduction, FP8 and the arrival stand-in.

Per-call HIP events (the library's kernel timing, chained: each call's end event taken by
its last kernel launch on the launch stream, each call timed from the previous call's end)
are taken inside the headline's timed region itself, so the roofline's kernel time is part of the timed step.  Prints one JSON line.  --profile-pass runs only one workload's
timed region (and a copy of known size that calibrates rocprofv3's byte counters).
"""

import argparse
import hashlib
import json
import os
import sys
import time

MFMA_PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense
MFMA_PEAK_FP8_TFLOPS = 5033.2   # dense fp8: twice the bf16 rate
HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
GEMM_SRC = os.path.join(ROOT, "chunked_tp_overlap_amd", "csrc", "gemm_bf16.hip")
REDUCE_SRC = os.path.join(ROOT, "chunked_tp_overlap_amd", "csrc", "reduce_partials.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
PROFILE_PASSES = ("gqa", "qkv", "fc1", "fc2", "reduce", "fp8", "arrival", "host")


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="minimum CPU-oracle baseline work (seconds)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--points", default=None,
                   help="with --profile-pass gqa: comma-separated T values of the sweep to run "
                        "instead of all 32")
    p.add_argument("--profile-pass", default=None, choices=PROFILE_PASSES,
                   help="for rocprofv3: run only this workload's timed region (with the "
                        "library's per-launch events), then a 1 GiB copy that calibrates the "
                        "byte counters, and print one JSON line (gqa: the headline sweep; qkv, "
                        "fc1: their microbatches; fc2: the slice GEMMs and reductions over its T "
                        "sweep; reduce: the fc2 reduction at T = 16384; fp8: the qkv step on an "
                        "fp8 buffer; arrival: separated arrival-stand-in calls of every mode; "
                        "host: separated qkv host-loop and device-loop calls)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def src_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


# ---- workloads ---------------------------------------------------------------------------

SCRATCH_BYTES = (64 << 20) + 256 * 1024  # partials of every split the library chooses + counters


def register_scratch(ub, torch, dev, h):
    t = torch.zeros(SCRATCH_BYTES // 2, dtype=torch.int16, device=dev)
    ub.ub_register_scratch(h, t, SCRATCH_BYTES)
    return t


class AgSweep:
    """An all-gather-side workload on one registered UserBuffer: a list of active T values,
    one ub_gemm_ag_chunked call per T."""

    def __init__(self, ub, wl, torch, np, dev, w, Ts):
        self.ub, self.torch, self.w, self.Ts = ub, torch, w, list(Ts)
        ra, rw, _ = w.seeds()
        log(f"generating {w.name}: capacity {w.capacity} x {w.hidden}, W {w.hidden} x {w.n_cols}")
        self.a_host = wl.activations(w, w.capacity, ra)
        self.w_host = wl.weights(w, rw)
        ub_bytes, _ = ub.ub_required_bytes(w.capacity, w.hidden, w.tp)
        self.ub_t = torch.from_numpy(self.a_host.view(np.int16).ravel()).to(dev)
        self.w_t = torch.from_numpy(self.w_host.view(np.int16)).to(dev)
        self.c_t = torch.empty((w.capacity, w.n_cols), dtype=torch.int16, device=dev)
        self.h = ub.ub_init(w.capacity, w.hidden, w.tp, ub.UB_DTYPE_BF16, self.ub_t, ub_bytes)
        # worker streams right after registration: they take hardware queues of their own
        ub.ub_prepare_streams(self.h, w.num_max_streams)
        # split-K scratch: lets the library sum the rows of an underfilled launch in K segments
        self.scratch = register_scratch(ub, torch, dev, self.h)
        self.stream = torch.cuda.current_stream()
        self.flops = sum(self.flop(T) for T in self.Ts)

    def flop(self, T):
        return 2.0 * T * self.w.hidden * self.w.n_cols

    def alg_bytes(self, T):
        w = self.w
        return 2.0 * (T * w.hidden + w.hidden * w.n_cols + T * w.n_cols)

    def cfg(self, atomic):
        w = self.w
        return self.ub.make_cfg(w.method, w.num_splits, w.num_max_streams, w.aggregate, atomic)

    def call(self, T, cfg):
        ub, w = self.ub, self.w
        ub.ub_set_active_shape(self.h, (T, w.hidden))
        ub.ub_gemm_ag_chunked(self.h, self.w_t, w.n_cols, w.n_cols, self.c_t, w.n_cols, cfg,
                              self.stream)

    def step(self, cfg):
        for T in self.Ts:
            self.call(T, cfg)

    def timed(self, cfg, steps, warmup, events=False):
        """Seconds per step over `steps` steps after `warmup` untimed ones.  events: the
        library's kernel timing is on during the timed steps (True or 1: an event pair per
        launch; 2: chained, one event per launch); returns (seconds, GEMM launch stats of
        those steps)."""
        ub, torch = self.ub, self.torch
        for _ in range(warmup):
            self.step(cfg)
        torch.cuda.synchronize()
        if events:
            ub.ub_set_kernel_timing(self.h, events)
            ub.ub_get_kernel_timing(self.h)
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step(cfg)
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / steps
        stats = None
        if events:
            stats, _ = ub.ub_get_kernel_timing(self.h)
            ub.ub_set_kernel_timing(self.h, False)
        return sec, stats

    def per_point(self, cfg, reps=20):
        """(T, median ms, min ms) per point: 5 warm-up calls, then `reps` calls timed one by
        one with HIP events on the launch stream."""
        out = []
        for T in self.Ts:
            med, best, _ = _call_stats(lambda: self.call(T, cfg), self.torch, self.stream, reps)
            out.append((T, med, best))
        return out

    def plans(self, cfg):
        """The tile plan of each point's call: (T, tile_m, tile_n, cut_row, tail_m, tail_n,
        seg_row, nseg, split, seg_tile_m, seg_tile_n)."""
        rows = []
        for T in self.Ts:
            self.call(T, cfg)
            rows.append((T,) + tuple(self.ub.ub_debug_last_plan(self.h, seg=True)))
        self.torch.cuda.synchronize()
        return rows

    def graph_replay(self, cfg, reps):
        """Seconds per step when one step (every T, each with its own active shape) is
        captured once in a HIP graph and replayed."""
        torch = self.torch
        s = torch.cuda.Stream()
        old = self.stream
        self.stream = s
        try:
            with torch.cuda.stream(s):
                self.step(cfg)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                self.step(cfg)
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                g.replay()
            torch.cuda.synchronize()
            return (time.perf_counter() - t0) / reps
        finally:
            self.stream = old

    def close(self):
        self.torch.cuda.synchronize()
        self.ub.ub_destroy(self.h)


def gqa_sweep(ub, wl, torch, np, dev):
    """The headline: the GQA bulk sweep's 32 grid points (1024 ... 32520; the extra point
    T = 32768 is reported with the secondary rows)."""
    return AgSweep(ub, wl, torch, np, dev, wl.gqa_bulk(), [T for T in wl.gqa_tokens() if T != 32768])


def qkv_step(ub, wl, torch, np, dev):
    w = wl.qkv()
    _, _, rt = w.seeds()
    Ts, _ = wl.qkv_pack_tokens(rt)
    return AgSweep(ub, wl, torch, np, dev, w, Ts)


def fc1_step(ub, wl, torch, np, dev):
    w = wl.fc1()
    _, _, rt = w.seeds()
    return AgSweep(ub, wl, torch, np, dev, w, wl.fc1_tokens(rt))


# ---- main --------------------------------------------------------------------------------

def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the work on a single MI355X; "
              f"--gpus {args.gpus} (WORLD_SIZE={world}) is not supported: the library has no "
              "multi-GPU path.", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import chunked_tp_overlap_amd.ub as ub
    from chunked_tp_overlap_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.profile_pass:
        fn = {"gqa": profile_ag, "qkv": profile_ag, "fc1": profile_ag, "fc2": profile_fc2,
              "reduce": profile_reduce, "fp8": profile_fp8, "arrival": profile_arrival,
              "host": profile_host}[args.profile_pass]
        res = fn(ub, wl, torch, np, dev, args)
        calibration_copy(torch, dev)
        print(json.dumps(res), flush=True)
        return

    g = gqa_sweep(ub, wl, torch, np, dev)
    primary = g.cfg(atomic=True)
    log(f"warmup {args.warmup}, timed {args.steps} steps of {len(g.Ts)} GQA points (atomic_gemm)")
    # chained kernel timing: one event per call, taken by the call's last kernel launch on the
    # launch stream; each call's time runs from the previous call's end event
    sec, stats = g.timed(primary, args.steps, args.warmup, events=2)
    tflops = g.flops / sec / 1e12
    log(f"primary: {sec * 1e3:.3f} ms/step, {tflops:.1f} TFLOP/s (chained per-call events on)")
    sec_clean, _ = g.timed(primary, args.steps, 1)
    log(f"same steps without events: {sec_clean * 1e3:.3f} ms/step")

    kernel_ms_per_step = stats["total_ms"] / args.steps
    achieved = stats["flops"] / (stats["total_ms"] / 1e3) / 1e12
    calls = stats["launches"]
    traffic, traffic_src = None, None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("src_hash") == src_hash(GEMM_SRC) and tr.get("workload") == "gqa":
            traffic = tr.get("bytes_per_call")
            traffic_src = tr.get("source")
    except (OSError, ValueError):
        pass
    roofline = {
        "bound": "mfma",
        "kernel": "gemm_bf16_* (device-side chunk loop; one call = one ping-pong/pipelined "
                  "launch, two when the plan cuts a nearly empty last round, plus a split-K "
                  "launch and its gemm_bf16_split_reduce for rows the plan sums in K segments)",
        "achieved": round(achieved, 2), "peak": MFMA_PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(achieved / MFMA_PEAK_BF16_TFLOPS, 4),
        "traffic": traffic,
        "traffic_note": (f"HBM bytes per call, mean over the sweep, from an earlier rocprofv3 "
                         f"FETCH_SIZE + WRITE_SIZE profile run of this same kernel source "
                         f"({traffic_src}); not measured in this run" if traffic
                         else "no counter pass of this kernel source"),
        "calls": calls,
        "avg_call_us": round(stats["total_ms"] * 1e3 / max(1, calls), 3),
        "avg_call_gflop": round(stats["flops"] / max(1, calls) / 1e9, 4),
        "algorithmic_bytes_per_call": round(stats["bytes"] / max(1, calls)),
        "kernel_ms_per_step": round(kernel_ms_per_step, 4),
        "timing": "HIP events on the launch stream inside the timed region, chained: each "
                  "GEMM call's end event recorded by its last kernel launch, each call's "
                  "time from the previous call's end event (the first from an event of its "
                  "own); kernel_ms_per_step <= ms_per_step",
    }

    w = g.w
    result = {
        "metric": "bf16 TFLOP/s of chunked AG/RS GEMM at active T; % of MFMA peak",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_mfma_peak": round(100 * tflops / MFMA_PEAK_BF16_TFLOPS, 2),
        "config": {
            "workload": "gqa_bulk_ag: GQA QKV column-parallel AG-GEMM, bulk mode, one [32768, 8192] "
                        "bf16 UserBuffer registered once, W [8192, 1280], tp 8, num_splits 8; one "
                        "step = the T sweep 1024, 2040, ..., 32520 (32 points, step 1016) with "
                        "ub_set_active_shape per point; device-side chunk loop",
            "capacity": w.capacity, "hidden": w.hidden, "n_cols": w.n_cols, "tp": w.tp,
            "method": w.method, "num_splits": w.num_splits, "num_max_streams": w.num_max_streams,
            "atomic_gemm": True, "points": len(g.Ts), "T_min": min(g.Ts), "T_max": max(g.Ts),
            "gflop_per_step": round(g.flops / 1e9, 2), "seed": w.seed,
        },
        "ms_per_step_without_events": round(sec_clean * 1e3, 4),
        "roofline": roofline,
    }
    per_pt = g.per_point(primary)
    result["per_point"] = {"columns": ["T", "tflops_median", "tflops_best", "plan"],
                           "note": "each point: 5 warm-up calls, 20 calls back to back, each timed between HIP events (one event per call); "
                                   "plan = tile_m x tile_n [cut row: tail tile] [split-K from row r: "
                                   "nseg segments on tile, summed in the kernel (r1) or by a second "
                                   "launch (r2)]",
                           "rows": []}
    plans = {p[0]: p[1:] for p in g.plans(primary)}
    for T, med, best in per_pt:
        plan = describe_plan(plans[T])
        result["per_point"]["rows"].append([T, round(g.flop(T) / med / 1e9, 1),
                                            round(g.flop(T) / best / 1e9, 1), plan])
    result["per_point"]["tflops_sum_flops_over_sum_medians"] = round(
        g.flops / (sum(m for _, m, _ in per_pt) / 1e3) / 1e12, 2)
    host_cfg = g.cfg(atomic=False)
    sec_h, _ = g.timed(host_cfg, max(2, args.steps // 4), 1)
    result["modes"] = {
        "atomic_gemm": {"tflops": round(tflops, 2), "ms_per_step": round(sec * 1e3, 4)},
        "host_loop_3_streams": {"tflops": round(g.flops / sec_h / 1e12, 2),
                                "ms_per_step": round(sec_h * 1e3, 4)},
    }
    result["graph_replay_tflops"] = {"atomic_gemm": round(g.flops / g.graph_replay(primary, 5) / 1e12, 2)}

    props = torch.cuda.get_device_properties(0)
    result["device"] = {"name": props.name, "cus": props.multi_processor_count,
                        "gcn_arch": getattr(props, "gcnArchName", ""),
                        "gemm_src_hash": src_hash(GEMM_SRC),
                        "gpu_max_hw_queues": os.environ.get("GPU_MAX_HW_QUEUES", "(runtime default)")}
    result["device_state"] = device_state(torch)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(g, args.cpu_seconds)
    g.close()
    del g

    if not args.no_secondary:
        result["secondary"] = secondary(ub, wl, torch, np, dev)
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


# ---- helpers -----------------------------------------------------------------------------

def device_state(torch):
    """The GPU's PCI address and socket power cap (amdsmi).  amdsmi's metrics table refreshes
    too slowly to sample the timed region, so no clock is read here: the effective clock of
    the profiled kernels is in their counter summaries under profiles/."""
    out = {"source": "amdsmi", "power_cap_w": None, "bdf": None}
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        p = torch.cuda.get_device_properties(0)
        bus = getattr(p, "pci_bus_id", None)
        h = None
        if bus is not None:
            want = f"{getattr(p, 'pci_domain_id', 0):04x}:{bus:02x}:{getattr(p, 'pci_device_id', 0):02x}"
            h = next((x for x in handles if amdsmi.amdsmi_get_gpu_device_bdf(x).lower().startswith(want)), None)
        if h is None and len(handles) == 1:
            h = handles[0]
        if h is None:
            raise RuntimeError(f"no amdsmi device matches cuda:0 among {len(handles)}")
        out["bdf"] = amdsmi.amdsmi_get_gpu_device_bdf(h)
        cap = amdsmi.amdsmi_get_power_cap_info(h).get("power_cap")
        out["power_cap_w"] = round(cap / 1e6 if cap and cap > 1e4 else cap, 1) if cap else None
    except Exception as e:  # noqa: BLE001 - the record is informational
        out["error"] = f"{type(e).__name__}: {e}"
    return out


def calibration_copy(torch, dev):
    """A plain device copy of exactly 1 GiB (2^29 int16 -> 2^29 int16): rocprofv3's
    FETCH_SIZE / WRITE_SIZE of it calibrate the counters of the profiled kernels."""
    src = torch.ones(1 << 29, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()


def _call_stats(fn, torch, stream, reps=20, warmup=5):
    """Per-call times (ms) of fn() from HIP events on `stream`: `warmup` untimed calls, then
    `reps` timed ones back to back, one event before the first and one after each (call i
    runs from event i to event i + 1; an event record costs a few us of GPU time, so one per
    call rather than a pair).  Returns (median, minimum, mean)."""
    for _ in range(warmup):
        fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for e in ev[1:]:
        fn()
        e.record(stream)
    torch.cuda.synchronize()
    t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))
    return t[len(t) // 2], t[0], sum(t) / len(t)


def _stats_row(flops, stats, peak):
    med, best, mean = stats
    return {"tflops": round(flops / med / 1e9, 2), "tflops_best": round(flops / best / 1e9, 2),
            "ms_median": round(med, 4), "ms_min": round(best, 4), "ms_mean": round(mean, 4),
            "pct_peak": round(100 * flops / med / 1e9 / peak, 2)}


def _time_calls(fn, torch, stream, reps):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _ag_rows(sw, cfg, label):
    """Per-microbatch medians of an AG workload and its aggregates (all, and T >= 4096)."""
    pts = sw.per_point(cfg)
    big = [(T, ms) for T, ms, _ in pts if T >= 4096]
    agg = lambda rows: (sum(sw.flop(T) for T, _ in rows) / (sum(ms for _, ms in rows) / 1e3) / 1e12
                        if rows else None)
    tf_all = agg([(T, ms) for T, ms, _ in pts])
    tf_big = agg(big)
    log(f"{label}: {tf_all:.1f} TFLOP/s over all points")
    return {"tflops_all": round(tf_all, 2),
            "tflops_T_ge_4096": round(tf_big, 2) if tf_big else None,
            "pct_peak_T_ge_4096": round(100 * tf_big / MFMA_PEAK_BF16_TFLOPS, 2) if tf_big else None}


# ---- secondary rows ----------------------------------------------------------------------

def secondary(ub, wl, torch, np, dev):
    out = {}
    stream = torch.cuda.current_stream()

    # GQA: the host loop per point, and the flagged extra point T = 32768
    g = AgSweep(ub, wl, torch, np, dev, wl.gqa_bulk(), wl.gqa_tokens())
    log("secondary gqa_bulk_ag host loop")
    res = {"host_loop_3_streams": _ag_rows(g, g.cfg(False), "gqa host loop")}
    med, best, _ = _call_stats(lambda: g.call(32768, g.cfg(True)), torch, g.stream)
    res["T_32768_atomic_gemm"] = {"tflops": round(g.flop(32768) / med / 1e9, 1),
                                  "plan": list(ub.ub_debug_last_plan(g.h))}
    out["gqa_bulk_ag"] = res
    g.close()
    del g

    # QKV: 32 THD microbatches of one step
    q = qkv_step(ub, wl, torch, np, dev)
    log("secondary qkv_ag")
    sec, qst = q.timed(q.cfg(True), 20, 5, events=2)
    sec_h, _ = q.timed(q.cfg(False), 10, 2)
    hl_ev = q.timed(q.cfg(False), 2, 0, events=True)[1]
    res = {"atomic_gemm": {"tflops_step": round(q.flops / sec / 1e12, 2), "ms_per_step": round(sec * 1e3, 4),
                           "kernel_tflops": round(qst["flops"] / (qst["total_ms"] / 1e3) / 1e12, 2),
                           **_ag_rows(q, q.cfg(True), "qkv device loop")},
           "host_loop_3_streams": {"tflops_step": round(q.flops / sec_h / 1e12, 2),
                                   "ms_per_step": round(sec_h * 1e3, 4),
                                   "avg_launch_us": round(hl_ev["total_ms"] * 1e3 / max(1, hl_ev["launches"]), 3)},
           "graph_replay_tflops": {"atomic_gemm": round(q.flops / q.graph_replay(q.cfg(True), 10) / 1e12, 2),
                                   "host_loop_3_streams": round(q.flops / q.graph_replay(q.cfg(False), 10) / 1e12, 2)},
           "microbatches": len(q.Ts), "T_mean": round(sum(q.Ts) / len(q.Ts), 1)}
    out["qkv_ag"] = res
    q.close()
    del q

    # fc1: SwiGLU gate+up, aggregate-2x, 16 microbatches
    f1 = fc1_step(ub, wl, torch, np, dev)
    log("secondary fc1_ag")
    out["fc1_ag"] = {"atomic_gemm": _ag_rows(f1, f1.cfg(True), "fc1 device loop"),
                     "host_loop_3_streams": _ag_rows(f1, f1.cfg(False), "fc1 host loop"),
                     "microbatches": len(f1.Ts),
                     "note": "per microbatch the median of 20 calls timed one by one; aggregates are "
                             "sum FLOPs / sum medians"}
    f1.close()
    del f1

    out["qkv_arrival"] = arrival(ub, wl, torch, np, dev)
    out["qkv_fp8"] = qkv_fp8(ub, wl, torch, np, dev)

    # fc2: row-parallel RS GEMM + reduction over the T sweep (pipeline, 4 chunks)
    w = wl.fc2()
    ra, rw, _ = w.seeds()
    log("secondary fc2_rs")
    ub_bytes, ws_bytes = ub.ub_required_bytes(w.capacity, w.hidden, w.tp)
    ub_t = torch.empty(w.capacity * w.hidden, dtype=torch.int16, device=dev)
    ws_t = torch.zeros(ws_bytes // 2, dtype=torch.int16, device=dev)  # counter region zero
    a_t = torch.from_numpy(wl.activations(w, w.capacity, ra).view(np.int16)).to(dev)
    w_t = torch.from_numpy(wl.weights(w, rw).view(np.int16)).to(dev)
    o_t = torch.empty((w.capacity, w.hidden), dtype=torch.int16, device=dev)
    flush = torch.empty(768 * 1024 * 1024 // 2, dtype=torch.int16, device=dev)
    h = ub.ub_init(w.capacity, w.hidden, w.tp, ub.UB_DTYPE_BF16, ub_t, ub_bytes, ws_t, ws_bytes)
    ub.ub_prepare_streams(h, w.num_max_streams)
    rows = []
    for T in wl.FC2_TOKENS:
        ub.ub_set_active_shape(h, (T, w.hidden))
        f = 2.0 * T * w.k * w.hidden
        row = {"T": T}
        variants = (("pipeline_3_streams", dict(atomic_gemm=False)),
                    ("atomic_gemm", dict(atomic_gemm=True)),
                    ("atomic_gemm_ring_order", dict(atomic_gemm=True, reduce_order="ring")),
                    ("fused_pipeline_3_streams", dict(atomic_gemm=False, fuse_reduce=True)),
                    ("fused_atomic_gemm", dict(atomic_gemm=True, fuse_reduce=True)))
        for name, kw in variants:
            cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, False, **kw)
            st = _call_stats(lambda: ub.ub_gemm_rs_chunked(h, a_t, w.k, w.k, w_t, w.hidden, o_t, w.hidden, cfg, stream),
                             torch, stream)
            row[name] = _stats_row(f, st, MFMA_PEAK_BF16_TFLOPS)
        rbytes = (w.tp + 1) * T * w.hidden * 2.0
        for order in ("ascending", "ring"):
            warm = _time_calls(lambda: ub.ub_reduce_partials(h, o_t, w.hidden, order, stream), torch, stream, 10)
            # honest: a 768 MB write between reductions evicts the 256 MB MALL
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            cold = []
            for _ in range(5):
                flush.fill_(1)
                e0.record(stream)
                ub.ub_reduce_partials(h, o_t, w.hidden, order, stream)
                e1.record(stream)
                torch.cuda.synchronize()
                cold.append(e0.elapsed_time(e1))
            cold_ms = sorted(cold)[len(cold) // 2]
            sfx = "" if order == "ascending" else "_ring"
            row.update({f"reduce{sfx}_gbs_warm": round(rbytes / warm / 1e6, 1),
                        f"reduce{sfx}_gbs_flushed": round(rbytes / cold_ms / 1e6, 1),
                        f"reduce{sfx}_pct_hbm_flushed": round(100 * rbytes / cold_ms / 1e6 / HBM_PEAK_GBS, 2)})
        rows.append(row)
    out["fc2_rs"] = rows

    # fc2 on E4M3 operands: A and W^T quantized once on the GPU (per-tensor 448 / amax),
    # then the same T sweep through ub_gemm_rs_chunked_fp8 (bf16 partials and sum)
    log("secondary fc2_rs_fp8")
    sa_q = 448.0 / float(a_t.view(torch.bfloat16).float().abs().max())
    sw_q = 448.0 / float(w_t.view(torch.bfloat16).float().abs().max())
    a8 = torch.empty((w.capacity, w.k), dtype=torch.uint8, device=dev)
    w8 = torch.empty((w.hidden, w.k), dtype=torch.uint8, device=dev)
    ub.ub_quantize_e4m3(a_t, w.k, a8, w.k, w.capacity, w.k, sa_q)
    ub.ub_quantize_e4m3(w_t.t().contiguous(), w.k, w8, w.k, w.hidden, w.k, sw_q)
    rows8 = []
    for T in wl.FC2_TOKENS:
        ub.ub_set_active_shape(h, (T, w.hidden))
        f = 2.0 * T * w.k * w.hidden
        row = {"T": T}
        for atomic in (False, True):
            cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, False, atomic)
            st = _call_stats(lambda: ub.ub_gemm_rs_chunked_fp8(h, a8, w.k, w.k, w8, w.k, 1.0 / sa_q, 1.0 / sw_q,
                                                               o_t, w.hidden, cfg, stream), torch, stream)
            row["atomic_gemm" if atomic else "pipeline_3_streams"] = _stats_row(f, st, MFMA_PEAK_FP8_TFLOPS)
        rows8.append(row)
    out["fc2_rs_fp8"] = {"rows": rows8, "note": "E4M3 A [T, 14336] and W [4096, 14336], per-tensor "
                         "scales, bf16 partials and sum; FLOPs 2 T K H per call; pct_peak of the fp8 peak"}
    ub.ub_destroy(h)
    del ub_t, ws_t, a_t, w_t, o_t, flush, a8, w8
    return out


def arrival(ub, wl, torch, np, dev):
    """Arrival stand-in on the QKV workload: the 7 non-local ring chunks are copied into the
    UserBuffer on a copy stream while the 8 chunk GEMMs (host loop, 3 streams) wait on their
    own chunk's event, or (modes *_device_loop) while the one device-side chunk loop's tiles
    wait on per-chunk flags written after each copy.  Sources: pinned host memory (SDMA
    over PCIe, about one xGMI link's rate), device memory by SDMA, device memory by the
    runtime's copy kernel (host loop only).  Reports the GEMMs alone, the deliveries alone,
    both overlapped, the fraction of the delivery time hidden behind the GEMMs, the overlap
    as a fraction of the shorter of the two, the time the call runs past the deliveries
    alone, and max(GEMMs, deliveries) / overlapped (1.0 when the shorter side is wholly
    hidden; the last chunk's GEMM can only follow its copy, so the bound is a little
    below 1).  The handle's streams (two workers and the copy stream) are created right
    after registration."""
    w = wl.qkv()
    ra, rw, _ = w.seeds()
    log("secondary qkv_arrival")
    ub_bytes, _ = ub.ub_required_bytes(w.capacity, w.hidden, w.tp)
    ub_t = torch.from_numpy(wl.activations(w, w.capacity, ra).view(np.int16).ravel()).to(dev)
    src = ub_t.clone()  # what the other ranks send: the same rows
    src_host = ub_t.cpu().pin_memory()
    w_t = torch.from_numpy(wl.weights(w, rw).view(np.int16)).to(dev)
    c_t = torch.empty((w.capacity, w.n_cols), dtype=torch.int16, device=dev)
    h = ub.ub_init(w.capacity, w.hidden, w.tp, ub.UB_DTYPE_BF16, ub_t, ub_bytes)
    ub.ub_prepare_streams(h, w.num_max_streams, copy_stream=True)
    scratch = register_scratch(ub, torch, dev, h)  # noqa: F841 (held while h is used)
    stream = torch.cuda.current_stream()
    res = []
    for T in (4096, 6144, 8192):
        ub.ub_set_active_shape(h, (T, w.hidden))
        row = {"T": T}
        for mode, use_ce, sb, atomic in (("host_pinned_sdma", True, src_host, False),
                                         ("device_sdma", True, src, False),
                                         ("device_copy_kernel", False, src, False),
                                         ("host_pinned_sdma_device_loop", True, src_host, True),
                                         ("device_sdma_device_loop", True, src, True)):
            cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, use_ce=use_ce, rank=0,
                              atomic_gemm=atomic)
            t_g = _time_calls(lambda: ub.ub_gemm_ag_chunked(h, w_t, w.n_cols, w.n_cols, c_t, w.n_cols, cfg, stream),
                              torch, stream, 10)
            t_c = _time_calls(lambda: ub.ub_deliver_chunks(h, sb, cfg, stream), torch, stream, 10)
            t_o = _time_calls(lambda: ub.ub_gemm_ag_arrival(h, sb, w_t, w.n_cols, w.n_cols, c_t, w.n_cols, cfg, stream),
                              torch, stream, 10)
            copy_bytes = 2.0 * (T - T // w.tp) * w.hidden
            row[mode] = {
                "gemm_ms": round(t_g, 4), "deliver_ms": round(t_c, 4), "overlapped_ms": round(t_o, 4),
                "deliver_gbs": round(copy_bytes / t_c / 1e6, 1),
                "hidden_fraction_of_delivery": round(max(0.0, min(1.0, (t_g + t_c - t_o) / t_c)), 3),
                "overlap_of_shorter": round(max(0.0, min(1.0, (t_g + t_c - t_o) / min(t_g, t_c))), 3),
                "exposed_after_delivery_ms": round(t_o - t_c, 4),
                "overlap_efficiency": round(max(t_g, t_c) / t_o, 3)}
        res.append(row)
    timeouts = ub.ub_arrival_timeouts(h)
    ub.ub_destroy(h)
    if timeouts:
        raise RuntimeError(f"arrival-gated device loop: {timeouts} tile waits timed out")
    return res


def qkv_fp8(ub, wl, torch, np, dev):
    """The QKV step on an FP8 (E4M3) UserBuffer: activations quantized into the buffer with
    a per-tensor scale, the weight quantized [N, K] through a scratch fp8 registration,
    then the 32 microbatches of one step through the device-side chunk loop."""
    w = wl.qkv()
    ra, rw, rt = w.seeds()
    Ts, _ = wl.qkv_pack_tokens(rt)
    log("secondary qkv_fp8")
    H, N = w.hidden, w.n_cols
    x = torch.from_numpy(wl.activations(w, w.capacity, ra).view(np.int16)).to(dev)
    wt = torch.from_numpy(wl.weights(w, rw).view(np.int16)).to(dev)
    sx = 448.0 / float(x.view(torch.bfloat16).float().abs().max())
    sw = 448.0 / float(wt.view(torch.bfloat16).float().abs().max())
    ub_t = torch.empty(w.capacity * H, dtype=torch.uint8, device=dev)
    h = ub.ub_init(w.capacity, H, w.tp, ub.UB_DTYPE_FP8_E4M3, ub_t, w.capacity * H)
    w8 = torch.empty(N * H, dtype=torch.uint8, device=dev)
    hw = ub.ub_init(N, H, 1, ub.UB_DTYPE_FP8_E4M3, w8, N * H)
    ub.ub_quantize_in(hw, wt.t().contiguous(), N, 0, sw)
    stream = torch.cuda.current_stream()
    q_ms = _time_calls(lambda: ub.ub_quantize_in(h, x, w.capacity, 0, sx), torch, stream, 10)
    cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, w.aggregate, True)
    c_t = torch.empty((w.capacity, N), dtype=torch.int16, device=dev)

    def step():
        for T in Ts:
            ub.ub_set_active_shape(h, (T, H))
            ub.ub_gemm_ag_chunked_fp8(h, w8, N, H, 1.0 / sx, 1.0 / sw, c_t, N, cfg, stream)

    for _ in range(10):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(20):
        step()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / 20
    flops = sum(2.0 * T * H * N for T in Ts)
    tf = flops / sec / 1e12
    ub.ub_destroy(h)
    ub.ub_destroy(hw)
    return {"tflops": round(tf, 2), "ms_per_step": round(sec * 1e3, 4),
            "pct_of_fp8_peak": round(100 * tf / MFMA_PEAK_FP8_TFLOPS, 2),
            "quantize_gbs": round(3.0 * w.capacity * H / q_ms / 1e6, 1),
            "note": "E4M3 operands, per-tensor scales, bf16 output; device-side chunk loop"}


# ---- profile passes (for rocprofv3) ------------------------------------------------------

def describe_plan(p):
    """(tile_m, tile_n, cut_row, tail_m, tail_n, seg_row, nseg, split, seg_tile_m,
    seg_tile_n) as text."""
    tm, tn, cut, sm, sn, seg_row, nseg, split, gm, gn = p
    out = []
    if seg_row != 0:
        out.append(f"{tm}x{tn}" + (f" cut {cut}: {sm}x{sn}" if cut >= 0 else ""))
    if nseg > 1:
        out.append(f"split-K from row {seg_row}: {nseg} x {gm}x{gn}" + (f" r{split}" if split else " fold"))
    return "; ".join(out)


def _call_dispatches(plan):
    """Kernel dispatches of one call from its plan (T, tile_m, tile_n, cut_row, tail_m,
    tail_n, seg_row, nseg, split, ...): the rows before seg_row launch once, or twice when
    cut; K-segmented rows once, or twice when their split sum is a separate launch."""
    cut, seg_row, nseg, split = plan[3], plan[6], plan[7], plan[8]
    n = 0
    if seg_row != 0:
        n += 2 if cut >= 0 else 1
    if nseg > 1:
        n += 2 if split == 2 else 1
    return n


def _dispatches(ub, sw, cfg):
    """Kernel dispatches of one step."""
    return sum(_call_dispatches(p) for p in sw.plans(cfg))


def profile_ag(ub, wl, torch, np, dev, args):
    """One AG workload's timed region in the device-side loop: warm-up steps, then timed
    steps with the library's per-launch events."""
    make = {"gqa": gqa_sweep, "qkv": qkv_step, "fc1": fc1_step}[args.profile_pass]
    sw = make(ub, wl, torch, np, dev)
    if args.points:
        keep = [int(x) for x in args.points.split(",")]
        sw.Ts = [T for T in keep if T <= sw.w.capacity]
        sw.flops = sum(sw.flop(T) for T in sw.Ts)
    cfg = sw.cfg(True)
    per_step = _dispatches(ub, sw, cfg)  # one untimed step that records the plans
    sec, stats = sw.timed(cfg, args.steps, args.warmup, events=True)
    alg = sum(sw.alg_bytes(T) for T in sw.Ts)
    out = {"profile_pass": args.profile_pass, "points": sw.Ts if args.points else "all",
           "ms_per_step": round(sec * 1e3, 4),
           "calls_per_step": len(sw.Ts), "dispatches_per_step": per_step,
           "timed_calls": args.steps * len(sw.Ts), "timed_dispatches": args.steps * per_step,
           "timed_gflop": round(args.steps * sw.flops / 1e9, 3),
           "timed_algorithmic_bytes": round(args.steps * alg),
           "hip_event_total_ms": round(stats["total_ms"], 4),
           "src_file": os.path.relpath(GEMM_SRC, ROOT), "src_hash": src_hash(GEMM_SRC)}
    sw.close()
    return out


def profile_fc2(ub, wl, torch, np, dev, args):
    """The fc2 RS GEMM in the device-side loop over its T sweep: per call one slice-GEMM
    launch (or two when its plan is cut) and one reduction launch; the timed region's GEMM
    and reduction launches are reported apart (keys gemm and reduce)."""
    w = wl.fc2()
    ra, rw, _ = w.seeds()
    ub_bytes, ws_bytes = ub.ub_required_bytes(w.capacity, w.hidden, w.tp)
    ub_t = torch.empty(w.capacity * w.hidden, dtype=torch.int16, device=dev)
    ws_t = torch.zeros(ws_bytes // 2, dtype=torch.int16, device=dev)
    a_t = torch.from_numpy(wl.activations(w, w.capacity, ra).view(np.int16)).to(dev)
    w_t = torch.from_numpy(wl.weights(w, rw).view(np.int16)).to(dev)
    o_t = torch.empty((w.capacity, w.hidden), dtype=torch.int16, device=dev)
    h = ub.ub_init(w.capacity, w.hidden, w.tp, ub.UB_DTYPE_BF16, ub_t, ub_bytes, ws_t, ws_bytes)
    stream = torch.cuda.current_stream()
    cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, False, True)
    Ts = list(wl.FC2_TOKENS)
    if args.points:
        Ts = [int(x) for x in args.points.split(",")]

    def step():
        for T in Ts:
            ub.ub_set_active_shape(h, (T, w.hidden))
            ub.ub_gemm_rs_chunked(h, a_t, w.k, w.k, w_t, w.hidden, o_t, w.hidden, cfg, stream)

    dispatches = 0
    for T in Ts:  # one untimed step that records the plans
        ub.ub_set_active_shape(h, (T, w.hidden))
        ub.ub_gemm_rs_chunked(h, a_t, w.k, w.k, w_t, w.hidden, o_t, w.hidden, cfg, stream)
        dispatches += 2 if ub.ub_debug_last_plan(h)[2] >= 0 else 1
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ub.ub_set_kernel_timing(h, True)
    ub.ub_get_kernel_timing(h)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / args.steps
    gs, rs = ub.ub_get_kernel_timing(h)
    ub.ub_set_kernel_timing(h, False)
    flops = sum(2.0 * T * w.k * w.hidden for T in Ts)
    out = {"profile_pass": "fc2", "T": Ts, "ms_per_step": round(sec * 1e3, 4),
           "tflops_step": round(flops / sec / 1e12, 2),
           "gemm": {"timed_calls": args.steps * len(Ts), "timed_dispatches": args.steps * dispatches,
                    "timed_gflop": round(args.steps * flops / 1e9, 3),
                    "timed_algorithmic_bytes": round(gs["bytes"]),
                    "hip_event_total_ms": round(gs["total_ms"], 4)},
           "reduce": {"timed_calls": args.steps * len(Ts), "timed_dispatches": args.steps * len(Ts),
                      "timed_algorithmic_bytes": round(rs["bytes"]),
                      "hip_event_total_ms": round(rs["total_ms"], 4)},
           "src_file": os.path.relpath(GEMM_SRC, ROOT), "src_hash": src_hash(GEMM_SRC)}
    ub.ub_destroy(h)
    return out


def profile_reduce(ub, wl, torch, np, dev, args):
    """The fc2 reduction at T = 16384 (8 bf16 partial slots of [16384, 4096]): warm-up
    launches, then timed launches with per-launch events; ascending order first, then ring
    order."""
    w = wl.fc2()
    ra, rw, _ = w.seeds()
    T = wl.FC2_TOKENS[-1]
    ub_bytes, ws_bytes = ub.ub_required_bytes(w.capacity, w.hidden, w.tp)
    ub_t = torch.empty(w.capacity * w.hidden, dtype=torch.int16, device=dev)
    ws_t = torch.zeros(ws_bytes // 2, dtype=torch.int16, device=dev)
    a_t = torch.from_numpy(wl.activations(w, T, ra).view(np.int16)).to(dev)
    w_t = torch.from_numpy(wl.weights(w, rw).view(np.int16)).to(dev)
    o_t = torch.empty((w.capacity, w.hidden), dtype=torch.int16, device=dev)
    h = ub.ub_init(w.capacity, w.hidden, w.tp, ub.UB_DTYPE_BF16, ub_t, ub_bytes, ws_t, ws_bytes)
    ub.ub_set_active_shape(h, (T, w.hidden))
    ub.ub_gemm_rs_chunked(h, a_t, w.k, w.k, w_t, w.hidden, o_t, w.hidden,
                          ub.make_cfg(w.method, w.num_splits, atomic_gemm=True))
    stream = torch.cuda.current_stream()
    out = {"profile_pass": "reduce", "T": T, "launches_per_order": args.warmup + args.steps}
    for order in ("ascending", "ring"):
        fn = lambda: ub.ub_reduce_partials(h, o_t, w.hidden, order, stream)
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ub.ub_set_kernel_timing(h, True)
        ub.ub_get_kernel_timing(h)
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        rs = ub.ub_get_kernel_timing(h)[1]
        ub.ub_set_kernel_timing(h, False)
        n = max(1, rs["launches"])
        out[order] = {"avg_launch_us_hip_events": round(rs["total_ms"] * 1e3 / n, 3),
                      "algorithmic_bytes_per_launch": round(rs["bytes"] / n),
                      "gbs_hip_events": round(rs["bytes"] / (rs["total_ms"] / 1e3) / 1e9, 1),
                      "timed_dispatches": args.steps,
                      "timed_algorithmic_bytes": round(rs["bytes"]),
                      "hip_event_total_ms": round(rs["total_ms"], 4)}
    out["src_file"] = os.path.relpath(REDUCE_SRC, ROOT)
    out["src_hash"] = src_hash(REDUCE_SRC)
    ub.ub_destroy(h)
    return out


def profile_host(ub, wl, torch, np, dev, args):
    """The pages' default schedule on qkv, for a rocprofv3 kernel trace: per T in (4096,
    6912, 8192), `steps` host-loop calls (8 ring chunks, one launch each, on 3 streams),
    then `steps` device-side-loop calls, each followed by a device synchronisation and a
    20 ms pause, so that every call stands alone on the timeline.  Prints the modes in
    trace order."""
    w = wl.qkv()
    ra, rw, _ = w.seeds()
    ub_bytes, _ = ub.ub_required_bytes(w.capacity, w.hidden, w.tp)
    ub_t = torch.from_numpy(wl.activations(w, w.capacity, ra).view(np.int16).ravel()).to(dev)
    w_t = torch.from_numpy(wl.weights(w, rw).view(np.int16)).to(dev)
    c_t = torch.empty((w.capacity, w.n_cols), dtype=torch.int16, device=dev)
    h = ub.ub_init(w.capacity, w.hidden, w.tp, ub.UB_DTYPE_BF16, ub_t, ub_bytes)
    ub.ub_prepare_streams(h, w.num_max_streams)
    scratch = register_scratch(ub, torch, dev, h)  # noqa: F841 (held while h is used)
    modes = []
    for T in (4096, 6912, 8192):
        ub.ub_set_active_shape(h, (T, w.hidden))
        for label, atomic in (("host_loop", False), ("device_loop", True)):
            cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, w.aggregate, atomic)
            call = lambda: ub.ub_gemm_ag_chunked(h, w_t, w.n_cols, w.n_cols, c_t, w.n_cols, cfg)
            call()  # untimed: first use of this shape
            torch.cuda.synchronize()
            time.sleep(0.02)
            for _ in range(args.steps):
                call()
                torch.cuda.synchronize()
                time.sleep(0.02)
            modes.append({"mode": f"{label} T={T}", "calls": args.steps + 1,
                          "gflop": round(2.0 * T * w.hidden * w.n_cols / 1e9, 3)})
    ub.ub_destroy(h)
    return {"profile_pass": "host", "workload": w.name, "chunks": w.tp,
            "streams": w.num_max_streams, "modes": modes,
            "gpu_max_hw_queues": os.environ.get("GPU_MAX_HW_QUEUES", "(runtime default)")}


ARRIVAL_MODES = (("host_loop_pinned_host", True, True, False),
                 ("host_loop_device_sdma", True, False, False),
                 ("host_loop_device_copy_kernel", False, False, False),
                 ("device_loop_pinned_host", True, True, True),
                 ("device_loop_device_sdma", True, False, True))


def profile_arrival(ub, wl, torch, np, dev, args):
    """Arrival stand-in on qkv at T = 8192 (ring, rank 0, 3 streams), for a rocprofv3
    kernel and memory-copy trace: per mode (host loop or device-side loop; pinned-host,
    device SDMA or copy-kernel source) `steps` calls, each followed by a device
    synchronisation and a 20 ms pause, so that every call stands alone on the timeline.
    Prints the modes in trace order."""
    w = wl.qkv()
    ra, rw, _ = w.seeds()
    T = w.capacity
    ub_bytes, _ = ub.ub_required_bytes(w.capacity, w.hidden, w.tp)
    ub_t = torch.from_numpy(wl.activations(w, w.capacity, ra).view(np.int16).ravel()).to(dev)
    src = ub_t.clone()
    src_host = ub_t.cpu().pin_memory()
    w_t = torch.from_numpy(wl.weights(w, rw).view(np.int16)).to(dev)
    c_t = torch.empty((w.capacity, w.n_cols), dtype=torch.int16, device=dev)
    h = ub.ub_init(w.capacity, w.hidden, w.tp, ub.UB_DTYPE_BF16, ub_t, ub_bytes)
    ub.ub_prepare_streams(h, w.num_max_streams, copy_stream=True)
    scratch = register_scratch(ub, torch, dev, h)  # noqa: F841 (held while h is used)
    ub.ub_set_active_shape(h, (T, w.hidden))
    torch.cuda.synchronize()
    time.sleep(0.05)  # the uploads above stand apart from the first call on the timeline
    modes = []
    for name, use_ce, host, atomic in ARRIVAL_MODES:
        cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, use_ce=use_ce, rank=0,
                          atomic_gemm=atomic)
        sb = src_host if host else src
        for _ in range(args.steps):
            ub.ub_gemm_ag_arrival(h, sb, w_t, w.n_cols, w.n_cols, c_t, w.n_cols, cfg)
            torch.cuda.synchronize()
            time.sleep(0.02)
        modes.append({"mode": name, "calls": args.steps})
    timeouts = ub.ub_arrival_timeouts(h)
    ub.ub_destroy(h)
    return {"profile_pass": "arrival", "T": T, "chunks": w.tp, "modes": modes,
            "timeouts": timeouts, "gpu_max_hw_queues": os.environ.get("GPU_MAX_HW_QUEUES", "(runtime default)")}


def profile_fp8(ub, wl, torch, np, dev, args):
    """The qkv step on an fp8 buffer (see qkv_fp8): warm-up steps, then timed steps with
    per-launch events."""
    w = wl.qkv()
    ra, rw, rt = w.seeds()
    Ts, _ = wl.qkv_pack_tokens(rt)
    H, N = w.hidden, w.n_cols
    x = torch.from_numpy(wl.activations(w, w.capacity, ra).view(np.int16)).to(dev)
    wt = torch.from_numpy(wl.weights(w, rw).view(np.int16)).to(dev)
    sx = 448.0 / float(x.view(torch.bfloat16).float().abs().max())
    sw = 448.0 / float(wt.view(torch.bfloat16).float().abs().max())
    ub_t = torch.empty(w.capacity * H, dtype=torch.uint8, device=dev)
    h = ub.ub_init(w.capacity, H, w.tp, ub.UB_DTYPE_FP8_E4M3, ub_t, w.capacity * H)
    w8 = torch.empty(N * H, dtype=torch.uint8, device=dev)
    hw = ub.ub_init(N, H, 1, ub.UB_DTYPE_FP8_E4M3, w8, N * H)
    ub.ub_quantize_in(hw, wt.t().contiguous(), N, 0, sw)
    ub.ub_quantize_in(h, x, w.capacity, 0, sx)
    cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, w.aggregate, True)
    c_t = torch.empty((w.capacity, N), dtype=torch.int16, device=dev)

    def step():
        for T in Ts:
            ub.ub_set_active_shape(h, (T, H))
            ub.ub_gemm_ag_chunked_fp8(h, w8, N, H, 1.0 / sx, 1.0 / sw, c_t, N, cfg)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ub.ub_set_kernel_timing(h, True)
    ub.ub_get_kernel_timing(h)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    gs = ub.ub_get_kernel_timing(h)[0]
    ub.ub_destroy(h)
    ub.ub_destroy(hw)
    src = os.path.join(ROOT, "chunked_tp_overlap_amd", "csrc", "gemm_fp8.hip")
    flops = sum(2.0 * T * H * N for T in Ts)
    return {"profile_pass": "fp8", "timed_dispatches": args.steps * len(Ts),
            "timed_gflop": round(args.steps * flops / 1e9, 3),
            "timed_algorithmic_bytes": round(gs["bytes"]), "hip_event_total_ms": round(gs["total_ms"], 4),
            "src_file": os.path.relpath(src, ROOT), "src_hash": src_hash(src)}


# ---- CPU baseline ------------------------------------------------------------------------

def cpu_baseline(sw, min_seconds):
    """The oracle as it stands, timed on the host cores over a bounded sample of the
    headline sweep: whole points of it (every 4th T, then the rest in order), until at
    least `min_seconds` of oracle work.  Each sampled point is also run on the GPU (outside
    the oracle's timing) and compared with the oracle's output element by element: the
    bit-equal fraction and the largest error as a fraction of the gate
    4e-3 * |a_row| * |w_col|."""
    import numpy as np

    from oracle import bf16 as ob
    from oracle import gemm as og
    from oracle import manager as om
    from oracle import plan as op

    ub, torch = sw.ub, sw.torch
    gpu_cfg = sw.cfg(True)
    w_cols = np.linalg.norm(ob.decode(sw.w_host), axis=0)
    parity = {"points": 0, "elements": 0, "bit_equal": 0, "max_err_over_gate": 0.0}
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = sum(i.get("num_threads", 0) for i in libs)
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
                         for i in libs) or "none found"
    except Exception:  # threadpoolctl missing: report the core count
        threads = os.cpu_count()
    w = sw.w
    model = om.UserBufferModel(w.capacity, w.hidden, w.tp)
    cfg = op.OverlapCfg(method=w.method, num_splits=w.num_splits,
                        num_max_streams=w.num_max_streams, aggregate=w.aggregate, atomic_gemm=True)
    c = np.empty((w.capacity, w.n_cols), np.uint16)
    order = sw.Ts[::4] + [T for i, T in enumerate(sw.Ts) if i % 4]
    flops = elapsed = 0.0
    done = []
    for T in order:
        if elapsed >= min_seconds:
            break
        model.set_active_shape((T, w.hidden))
        model.fill_active(sw.a_host[:T])
        t0 = time.perf_counter()
        og.ag_chunked(model, sw.w_host, w.n_cols, w.n_cols, c, w.n_cols, cfg)
        elapsed += time.perf_counter() - t0
        flops += sw.flop(T)
        done.append(T)
        sw.call(T, gpu_cfg)  # parity of this point, untimed
        torch.cuda.synchronize()
        g = sw.c_t[:T].cpu().numpy().view(np.uint16)
        err = np.abs(ob.decode(g) - ob.decode(c[:T]))
        gate = 4e-3 * np.outer(np.linalg.norm(ob.decode(sw.a_host[:T]), axis=1), w_cols)
        parity["points"] += 1
        parity["elements"] += int(g.size)
        parity["bit_equal"] += int(np.sum(g == c[:T]))
        parity["max_err_over_gate"] = max(parity["max_err_over_gate"], float(np.max(err / gate)))
        log(f"cpu oracle: T={T}, {elapsed:.1f} s so far")
    return {"value": round(flops / elapsed / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(done)} points of the GQA sweep (T = {done}), whole points, numpy fp64 "
                      f"chunked GEMM + bf16 RNE over the capacity-buffer model, {elapsed:.1f} s",
            "host_cpus": os.cpu_count(), "blas": blas,
            "parity": {"points": parity["points"], "elements": parity["elements"],
                       "bit_equal_fraction": round(parity["bit_equal"] / max(1, parity["elements"]), 5),
                       "max_err_over_gate": round(parity["max_err_over_gate"], 5),
                       "note": "device-side chunk loop vs the oracle on every sampled point"}}


if __name__ == "__main__":
    main()
