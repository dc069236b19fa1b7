#!/usr/bin/env python3
"""Benchmark of the chunked tensor-parallel overlap GEMMs on one MI355X.

Metric: bf16 TFLOP/s of the chunked AG/RS GEMM at the active T, and its fraction of the
dense bf16 MFMA peak.  One step = one pass of the hot path over one batch of the QKV
workload: for each of its 32 THD microbatches, set the active shape [T, 4096] on the one
capacity-8192 UserBuffer and run the chunked all-gather-side GEMM (W [4096, 1536], ring
exchange over tp = 8 chunks).  FLOPs are algorithmic: 2 * T * 4096 * 1536 per microbatch,
active T only.  Inputs are seeded synthetic draws already resident in HBM when the timed
region starts.

The primary schedule is the device-side chunk loop (option atomic_gemm: one launch per
call whose workgroups walk the 8 ring chunks in ring order); the host loop of per-chunk
launches on min(8, 3) streams is measured as well and reported under "modes".

Prints one JSON line.  --profile-pass [qkv|reduce|fp8] runs only one kernel's timed region
(and a copy kernel of known size) for rocprofv3.
"""

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

MFMA_PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense
MFMA_PEAK_FP8_TFLOPS = 5033.2   # dense fp8: twice the bf16 rate
HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
GEMM_SRC = os.path.join(ROOT, "chunked_tp_overlap_amd", "csrc", "gemm_bf16.hip")
REDUCE_SRC = os.path.join(ROOT, "chunked_tp_overlap_amd", "csrc", "reduce_partials.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum CPU-oracle baseline work (seconds)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--profile-pass", nargs="?", const="qkv", default=None,
                   choices=["qkv", "reduce", "fp8", "arrival"],
                   help="for rocprofv3: run only one kernel's timed region and its per-launch "
                        "timing pass (qkv: the primary bf16 GEMM; reduce: the fc2 reduction at "
                        "T = 16384; fp8: the qkv step on an fp8 buffer), then a 1 GiB copy that "
                        "calibrates the byte counters; arrival: separated arrival-stand-in calls "
                        "of every mode, for a timeline; print one JSON line")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def src_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


class Qkv:
    """The QKV workload on one registered UserBuffer."""

    def __init__(self, ub, wl, torch, np, dev):
        self.ub, self.torch = ub, torch
        w = self.w = wl.qkv()
        ra, rw, rt = w.seeds()
        self.Ts, _ = wl.qkv_pack_tokens(rt)
        log(f"generating inputs: capacity {w.capacity} x {w.hidden}, W {w.hidden} x {w.n_cols}")
        self.a_host = wl.activations(w, w.capacity, ra)
        self.w_host = wl.weights(w, rw)
        ub_bytes, _ = ub.ub_required_bytes(w.capacity, w.hidden, w.tp)
        self.ub_t = torch.from_numpy(self.a_host.view(np.int16).ravel()).to(dev)
        self.w_t = torch.from_numpy(self.w_host.view(np.int16)).to(dev)
        self.c_t = torch.empty((w.capacity, w.n_cols), dtype=torch.int16, device=dev)
        self.h = ub.ub_init(w.capacity, w.hidden, w.tp, ub.UB_DTYPE_BF16, self.ub_t, ub_bytes)
        self.flops = sum(2.0 * T * w.hidden * w.n_cols for T in self.Ts)
        self.stream = torch.cuda.current_stream()

    def cfg(self, atomic):
        w = self.w
        return self.ub.make_cfg(w.method, w.num_splits, w.num_max_streams, w.aggregate, atomic)

    def step(self, cfg):
        ub, w = self.ub, self.w
        for T in self.Ts:
            ub.ub_set_active_shape(self.h, (T, w.hidden))
            ub.ub_gemm_ag_chunked(self.h, self.w_t, w.n_cols, w.n_cols, self.c_t, w.n_cols, cfg,
                                  self.stream)

    def timed(self, cfg, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step(cfg)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step(cfg)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def graph_replay(self, cfg, reps):
        """Seconds per step when one step (32 microbatches, each with its own active
        shape) is captured once in a HIP graph and replayed."""
        torch = self.torch
        s = torch.cuda.Stream()
        old = self.stream
        self.stream = s
        try:
            with torch.cuda.stream(s):
                self.step(cfg)  # warm: streams and events exist before capture
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

    def per_microbatch(self, cfg, reps=20):
        """(T, median ms, min ms) per microbatch: 5 warm-up calls, then `reps` calls timed
        one by one with HIP events on the launch stream."""
        ub, w = self.ub, self.w
        out = []
        for T in self.Ts:
            ub.ub_set_active_shape(self.h, (T, w.hidden))
            med, best, _ = _call_stats(
                lambda: ub.ub_gemm_ag_chunked(self.h, self.w_t, w.n_cols, w.n_cols, self.c_t, w.n_cols,
                                              cfg, self.stream), self.torch, self.stream, reps)
            out.append((T, med, best))
        return out


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the work on a single MI355X; "
              f"--gpus {args.gpus} (WORLD_SIZE={world}) is not supported: the library has no "
              "multi-GPU path.", file=sys.stderr, flush=True)
        sys.exit(2)

    # A handle's host-loop and arrival schedules use up to four streams (the caller's, two
    # workers, the copy stream).  HIP maps a process's streams onto GPU_MAX_HW_QUEUES
    # hardware queues (default 4); streams that share a queue run in issue order, which
    # serialises the arrival copies with the GEMMs once the benchmark's earlier sections
    # have created streams of their own.  At least eight queues keep them apart.  Set
    # before HIP initialises; a larger setting in the environment is kept.
    try:
        queues = int(os.environ.get("GPU_MAX_HW_QUEUES", "4"))
    except ValueError:
        queues = 4
    os.environ["GPU_MAX_HW_QUEUES"] = str(max(queues, 8))
    import numpy as np
    import torch

    import chunked_tp_overlap_amd.ub as ub
    from chunked_tp_overlap_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.profile_pass in ("reduce", "fp8", "arrival"):
        fn = {"reduce": profile_reduce, "fp8": profile_fp8, "arrival": profile_arrival}[args.profile_pass]
        res = fn(ub, wl, torch, np, dev, args.steps, args.warmup)
        calibration_copy(torch, dev)
        print(json.dumps(res), flush=True)
        return
    q = Qkv(ub, wl, torch, np, dev)
    primary = q.cfg(atomic=True)
    # One host-loop call first, so that the handle's worker streams exist before the
    # benchmark's graph captures start using torch's stream pool.  HIP places each stream
    # on one of GPU_MAX_HW_QUEUES hardware queues, and streams that share a queue run in
    # issue order.  When the worker streams were first created inside the capture code, the
    # eager host loop measured ~320 TFLOP/s instead of ~440, with the same kernels.
    q.step(q.cfg(atomic=False))
    torch.cuda.synchronize()

    log(f"warmup {args.warmup}, timed {args.steps} steps of {len(q.Ts)} microbatches (atomic_gemm)")
    sec = q.timed(primary, args.steps, args.warmup)
    tflops = q.flops / sec / 1e12
    log(f"primary: {sec * 1e3:.3f} ms/step, {tflops:.1f} TFLOP/s")

    # the same timed region again with per-launch HIP events on the launch stream
    ub.ub_set_kernel_timing(q.h, True)
    ub.ub_get_kernel_timing(q.h)
    sec_i = q.timed(primary, args.steps, 0)
    gemm_stats, _ = ub.ub_get_kernel_timing(q.h)
    ub.ub_set_kernel_timing(q.h, False)
    g_ach = gemm_stats["flops"] / (gemm_stats["total_ms"] / 1e3) / 1e12
    avg_launch_us = gemm_stats["total_ms"] * 1e3 / max(1, gemm_stats["launches"])

    if args.profile_pass:
        calibration_copy(torch, dev)
        ub.ub_destroy(q.h)
        print(json.dumps({"profile_pass": "qkv", "ms_per_step": round(sec * 1e3, 4),
                          "launches_per_step": len(q.Ts),
                          "launches": (args.warmup + 2 * args.steps) * len(q.Ts),
                          "timed_launches": 2 * args.steps * len(q.Ts),
                          "avg_launch_us_hip_events": round(avg_launch_us, 3),
                          "avg_launch_gflop": round(gemm_stats["flops"] / max(1, gemm_stats["launches"]) / 1e9, 4),
                          "algorithmic_bytes_per_launch": round(gemm_stats["bytes"] / max(1, gemm_stats["launches"])),
                          "src_file": os.path.relpath(GEMM_SRC, ROOT),
                          "src_hash": src_hash(GEMM_SRC)}), flush=True)
        return

    per_mb = q.per_microbatch(primary)
    fl = lambda T: 2.0 * T * q.w.hidden * q.w.n_cols
    big = [(T, med) for T, med, _ in per_mb if T >= 4096]
    agg_ge4096 = sum(fl(T) for T, _ in big) / (sum(ms for _, ms in big) / 1e3) / 1e12
    agg_all = sum(fl(T) for T, _, _ in per_mb) / (sum(ms for _, ms, _ in per_mb) / 1e3) / 1e12

    host_cfg = q.cfg(atomic=False)
    graph = {}
    for name, cfg in (("atomic_gemm", primary), ("host_loop_3_streams", host_cfg)):
        graph[name] = round(q.flops / q.graph_replay(cfg, args.steps) / 1e12, 2)
    sec_h = q.timed(host_cfg, max(2, args.steps // 2), 1)
    ub.ub_set_kernel_timing(q.h, True)
    ub.ub_get_kernel_timing(q.h)
    q.timed(host_cfg, 2, 0)
    host_stats, _ = ub.ub_get_kernel_timing(q.h)
    ub.ub_set_kernel_timing(q.h, False)

    traffic, util = None, None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("src_hash") == src_hash(GEMM_SRC):
            traffic = tr.get("qkv_gemm_bytes_per_launch")
            util = tr.get("util")
    except (OSError, ValueError):
        pass

    roofline = {
        "bound": "mfma", "kernel": "gemm_bf16_pingpong (device-side chunk loop, one launch per call)",
        "achieved": round(g_ach, 2), "peak": MFMA_PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(g_ach / MFMA_PEAK_BF16_TFLOPS, 4), "traffic": traffic,
        "launches": gemm_stats["launches"],
        "avg_launch_us": round(avg_launch_us, 3),
        "avg_launch_gflop": round(gemm_stats["flops"] / max(1, gemm_stats["launches"]) / 1e9, 4),
        "algorithmic_bytes_per_launch": round(gemm_stats["bytes"] / max(1, gemm_stats["launches"])),
        "measured_pass_ms_per_step": round(sec_i * 1e3, 4),
    }
    if util:
        # from the committed counter pass of the same kernel source (rocprofv3 --pmc
        # GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES): the effective clock,
        # the mean number of CUs holding a tile, and how busy their matrix cores are
        roofline["counters"] = util

    w = q.w
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
            "workload": "qkv_ag: column-parallel AG-GEMM over a [8192, 4096] bf16 UserBuffer, "
                        "W [4096, 1536], tp 8, ring exchange (8 chunks), 32 THD microbatches "
                        "per step, device-side chunk loop",
            "capacity": w.capacity, "hidden": w.hidden, "n_cols": w.n_cols, "tp": w.tp,
            "method": w.method, "num_splits": w.num_splits, "num_max_streams": w.num_max_streams,
            "atomic_gemm": True, "microbatches": len(q.Ts), "T_min": min(q.Ts), "T_max": max(q.Ts),
            "T_mean": round(sum(q.Ts) / len(q.Ts), 1), "gflop_per_step": round(q.flops / 1e9, 2),
            "seed": w.seed,
        },
        "tflops_T_ge_4096_per_microbatch_aggregate": round(agg_ge4096, 3),
        "tflops_all_per_microbatch_aggregate": round(agg_all, 3),
        "per_microbatch": {"columns": ["T", "tflops_median", "tflops_best"],
                           "note": "each microbatch: 5 warm-up calls, 20 calls timed one by one (HIP events)",
                           "rows": [[T, round(fl(T) / med / 1e9, 1), round(fl(T) / best / 1e9, 1)]
                                    for T, med, best in per_mb]},
        "graph_replay_tflops": graph,
        "modes": {
            "atomic_gemm": {"tflops": round(tflops, 2), "ms_per_step": round(sec * 1e3, 4)},
            "host_loop_3_streams": {
                "tflops": round(q.flops / sec_h / 1e12, 2), "ms_per_step": round(sec_h * 1e3, 4),
                "avg_launch_us": round(host_stats["total_ms"] * 1e3 / max(1, host_stats["launches"]), 3),
                "per_launch_tflops": round(host_stats["flops"] / max(1e-9, host_stats["total_ms"] / 1e3) / 1e12, 2)},
        },
        "roofline": roofline,
    }

    props = torch.cuda.get_device_properties(0)
    result["device"] = {"name": props.name, "cus": props.multi_processor_count,
                        "gcn_arch": getattr(props, "gcnArchName", ""),
                        "gemm_src_hash": src_hash(GEMM_SRC),
                        "gpu_max_hw_queues": os.environ.get("GPU_MAX_HW_QUEUES")}
    result["device_state"] = device_state(torch)

    if not args.no_secondary:
        result["secondary"] = secondary(ub, wl, torch, np, dev)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(q, args.cpu_seconds)

    ub.ub_destroy(q.h)
    busy = int(round(util["busy_cus_mean"])) if util and util.get("busy_cus_mean") else 142
    ceiling = mfma_ceiling(busy, props.multi_processor_count)
    if ceiling:
        burst = ceiling.get("bursts_tflops_at_busy_cus")
        if burst:
            ceiling["achieved_over_bursts_ceiling"] = round(g_ach / burst, 4)
        fp8 = (result.get("secondary") or {}).get("qkv_fp8")
        burst8 = ceiling.get("fp8_bursts_tflops_at_busy_cus")
        if fp8 and burst8:
            # the FP8 qkv step's rate (launch gaps included) over the FP8 MFMAs' own ceiling
            ceiling["fp8_step_over_fp8_bursts_ceiling"] = round(fp8["tflops"] / burst8, 4)
        roofline["mfma_ceiling"] = ceiling
    print(json.dumps(result), flush=True)


def mfma_ceiling(busy_cus, all_cus):
    """The matrix cores' own ceiling under the power limit, from the calibration program
    ``lib/mfma_ceiling`` (the bf16 GEMM's MFMA sequence in its 16x16x32 and 32x32x16 forms
    and the FP8 GEMM's, on register operands, no memory work),
    run as a child process: 32 launches of ~80 us back to back (the qkv step's launch
    pattern) and one sustained launch, on `busy_cus` CUs and on all of them, with the clock
    each ran at.  None if the program is missing or fails."""
    exe = os.path.join(ROOT, "chunked_tp_overlap_amd", "lib", "mfma_ceiling")
    if not os.path.exists(exe):
        log("mfma_ceiling program not built; skipping the ceiling")
        return None
    cus = sorted({max(1, min(busy_cus, all_cus)), all_cus})
    cmd = [exe, "0.5", *[str(c) for c in cus]]
    try:
        res = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    except subprocess.TimeoutExpired:
        log("mfma_ceiling timed out")
        return None
    if res.returncode != 0:
        log(f"mfma_ceiling failed ({res.returncode}): {res.stderr.strip()[-300:]}")
        return None
    rows = [json.loads(ln) for ln in res.stdout.splitlines() if ln.startswith("{")]

    def burst(kind):
        b = [r["bursts_32x80us"]["tflops"] for r in rows
             if r.get("kind") == kind and r["cus"] == cus[0] and r["waves_per_simd"] == 2]
        return b[0] if b else None

    # the bf16 GEMM issues v_mfma_f32_16x16x32_bf16 (kind "bf16_16x16x32"); the 32x32x16
    # form ("bf16") is kept for reference
    return {"program": "chunked_tp_overlap_amd/lib/mfma_ceiling " + " ".join(cmd[1:]),
            "busy_cus": cus[0], "bursts_tflops_at_busy_cus": burst("bf16_16x16x32"),
            "bursts_32x32x16_tflops_at_busy_cus": burst("bf16"),
            "fp8_bursts_tflops_at_busy_cus": burst("fp8"), "rows": rows}


def device_state(torch):
    """The GPU's PCI address and socket power cap (amdsmi).  amdsmi's metrics table refreshes
    too slowly to sample the ~0.1 s timed region, so no clock is read here: the effective
    clock of the timed kernel comes from the counter pass (roofline.counters)."""
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


def _instrumented(ub, h, torch, fn, reps, kind):
    """Run fn() reps times with the library's per-launch HIP events; (launches, mean us,
    mean GFLOP, mean algorithmic bytes) of launches of `kind` (0 GEMM, 1 reduction)."""
    ub.ub_set_kernel_timing(h, True)
    ub.ub_get_kernel_timing(h)
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    stats = ub.ub_get_kernel_timing(h)[kind]
    ub.ub_set_kernel_timing(h, False)
    n = max(1, stats["launches"])
    return stats["launches"], stats["total_ms"] * 1e3 / n, stats["flops"] / n / 1e9, stats["bytes"] / n


def profile_reduce(ub, wl, torch, np, dev, steps, warmup):
    """The fc2 reduction at T = 16384 (8 bf16 partial slots of [16384, 4096]): warm-up
    launches, timed launches, then the same with per-launch events; ascending order first,
    then ring order."""
    w = wl.fc2()
    ra, rw, _ = w.seeds()
    T = wl.FC2_TOKENS[-1]
    ub_bytes, ws_bytes = ub.ub_required_bytes(w.capacity, w.hidden, w.tp)
    ub_t = torch.empty(w.capacity * w.hidden, dtype=torch.int16, device=dev)
    ws_t = torch.empty(w.tp * w.capacity * w.hidden, dtype=torch.int16, device=dev)
    a_t = torch.from_numpy(wl.activations(w, T, ra).view(np.int16)).to(dev)
    w_t = torch.from_numpy(wl.weights(w, rw).view(np.int16)).to(dev)
    o_t = torch.empty((w.capacity, w.hidden), dtype=torch.int16, device=dev)
    h = ub.ub_init(w.capacity, w.hidden, w.tp, ub.UB_DTYPE_BF16, ub_t, ub_bytes, ws_t, ws_bytes)
    ub.ub_set_active_shape(h, (T, w.hidden))
    ub.ub_gemm_rs_chunked(h, a_t, w.k, w.k, w_t, w.hidden, o_t, w.hidden,
                          ub.make_cfg(w.method, w.num_splits, atomic_gemm=True))
    stream = torch.cuda.current_stream()
    out = {"profile_pass": "reduce", "T": T, "launches_per_order": warmup + 2 * steps}
    for order in ("ascending", "ring"):
        fn = lambda: ub.ub_reduce_partials(h, o_t, w.hidden, order, stream)
        for _ in range(warmup + steps):
            fn()
        n, us, _, nbytes = _instrumented(ub, h, torch, fn, steps, 1)
        out[order] = {"avg_launch_us_hip_events": round(us, 3), "algorithmic_bytes_per_launch": round(nbytes),
                      "gbs_hip_events": round(nbytes / us / 1e3, 1), "timed_launches": 2 * steps}
    out["src_file"] = os.path.relpath(REDUCE_SRC, ROOT)
    out["src_hash"] = src_hash(REDUCE_SRC)
    ub.ub_destroy(h)
    return out


ARRIVAL_MODES = (("host_loop_pinned_host", True, True, False),
                 ("host_loop_device_sdma", True, False, False),
                 ("host_loop_device_copy_kernel", False, False, False),
                 ("device_loop_pinned_host", True, True, True),
                 ("device_loop_device_sdma", True, False, True))


def profile_arrival(ub, wl, torch, np, dev, steps, warmup):
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
    ub.ub_set_active_shape(h, (T, w.hidden))
    torch.cuda.synchronize()
    time.sleep(0.05)  # the uploads above stand apart from the first call on the timeline
    modes = []
    for name, use_ce, host, atomic in ARRIVAL_MODES:
        cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, use_ce=use_ce, rank=0,
                          atomic_gemm=atomic)
        sb = src_host if host else src
        for _ in range(steps):
            ub.ub_gemm_ag_arrival(h, sb, w_t, w.n_cols, w.n_cols, c_t, w.n_cols, cfg)
            torch.cuda.synchronize()
            time.sleep(0.02)
        modes.append({"mode": name, "calls": steps})
    timeouts = ub.ub_arrival_timeouts(h)
    ub.ub_destroy(h)
    return {"profile_pass": "arrival", "T": T, "chunks": w.tp, "modes": modes,
            "timeouts": timeouts, "gpu_max_hw_queues": os.environ.get("GPU_MAX_HW_QUEUES")}


def profile_fp8(ub, wl, torch, np, dev, steps, warmup):
    """The qkv step on an fp8 buffer (see qkv_fp8): warm-up steps, timed steps, then the
    same with per-launch events."""
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

    for _ in range(warmup + steps):
        step()
    n, us, gflop, nbytes = _instrumented(ub, h, torch, step, steps, 0)
    ub.ub_destroy(h)
    ub.ub_destroy(hw)
    src = os.path.join(ROOT, "chunked_tp_overlap_amd", "csrc", "gemm_fp8.hip")
    return {"profile_pass": "fp8", "launches": (warmup + 2 * steps) * len(Ts),
            "timed_launches": 2 * steps * len(Ts), "avg_launch_us_hip_events": round(us, 3),
            "avg_launch_gflop": round(gflop, 4), "algorithmic_bytes_per_launch": round(nbytes),
            "src_file": os.path.relpath(src, ROOT), "src_hash": src_hash(src)}


def _call_stats(fn, torch, stream, reps=20, warmup=5):
    """Per-call times (ms) of fn() with HIP events around each call on `stream`: `warmup`
    untimed calls, then `reps` timed ones.  Returns (median, minimum, mean)."""
    for _ in range(warmup):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
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


def secondary(ub, wl, torch, np, dev):
    out = {}
    stream = torch.cuda.current_stream()

    # fc1: SwiGLU gate+up, aggregate-2x, 16 microbatches
    w = wl.fc1()
    ra, rw, rt = w.seeds()
    Ts = wl.fc1_tokens(rt)
    log("secondary fc1_ag")
    ub_bytes, _ = ub.ub_required_bytes(w.capacity, w.hidden, w.tp)
    ub_t = torch.from_numpy(wl.activations(w, w.capacity, ra).view(np.int16).ravel()).to(dev)
    w_t = torch.from_numpy(wl.weights(w, rw).view(np.int16)).to(dev)
    c_t = torch.empty((w.capacity, w.n_cols), dtype=torch.int16, device=dev)
    h = ub.ub_init(w.capacity, w.hidden, w.tp, ub.UB_DTYPE_BF16, ub_t, ub_bytes)
    res = {}
    for atomic in (True, False):
        cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, w.aggregate, atomic)
        tot_f = tot_ms = big_f = big_ms = 0.0
        for T in Ts:
            ub.ub_set_active_shape(h, (T, w.hidden))
            ms, _, _ = _call_stats(lambda: ub.ub_gemm_ag_chunked(h, w_t, w.n_cols, w.n_cols, c_t, w.n_cols, cfg, stream),
                                   torch, stream)
            f = 2.0 * T * w.hidden * w.n_cols
            tot_f += f
            tot_ms += ms
            if T >= 4096:
                big_f += f
                big_ms += ms
        res["atomic_gemm" if atomic else "host_loop"] = {
            "tflops_all": round(tot_f / tot_ms / 1e9, 2),
            "tflops_T_ge_4096": round(big_f / big_ms / 1e9, 2) if big_ms else None,
            "pct_peak_T_ge_4096": round(100 * big_f / big_ms / 1e9 / MFMA_PEAK_BF16_TFLOPS, 2) if big_ms else None}
    res["microbatches"] = len(Ts)
    res["note"] = "per microbatch the median of 20 calls timed one by one; aggregates are sum FLOPs / sum medians"
    out["fc1_ag"] = res
    ub.ub_destroy(h)
    del ub_t, w_t, c_t

    out["qkv_arrival"] = arrival(ub, wl, torch, np, dev)
    out["qkv_fp8"] = qkv_fp8(ub, wl, torch, np, dev)

    # fc2: row-parallel RS GEMM + reduction over the T sweep (pipeline, 4 chunks)
    w = wl.fc2()
    ra, rw, _ = w.seeds()
    log("secondary fc2_rs")
    ub_bytes, ws_bytes = ub.ub_required_bytes(w.capacity, w.hidden, w.tp)
    ub_t = torch.empty(w.capacity * w.hidden, dtype=torch.int16, device=dev)
    ws_t = torch.empty(w.tp * w.capacity * w.hidden, dtype=torch.int16, device=dev)
    a_t = torch.from_numpy(wl.activations(w, w.capacity, ra).view(np.int16)).to(dev)
    w_t = torch.from_numpy(wl.weights(w, rw).view(np.int16)).to(dev)
    o_t = torch.empty((w.capacity, w.hidden), dtype=torch.int16, device=dev)
    flush = torch.empty(768 * 1024 * 1024 // 2, dtype=torch.int16, device=dev)
    h = ub.ub_init(w.capacity, w.hidden, w.tp, ub.UB_DTYPE_BF16, ub_t, ub_bytes, ws_t, ws_bytes)
    rows = []
    for T in wl.FC2_TOKENS:
        ub.ub_set_active_shape(h, (T, w.hidden))
        f = 2.0 * T * w.k * w.hidden
        row = {"T": T}
        for atomic in (False, True):
            cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, False, atomic)
            st = _call_stats(lambda: ub.ub_gemm_rs_chunked(h, a_t, w.k, w.k, w_t, w.hidden, o_t, w.hidden, cfg, stream),
                             torch, stream)
            row["atomic_gemm" if atomic else "pipeline_3_streams"] = _stats_row(f, st, MFMA_PEAK_BF16_TFLOPS)
        cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, False, True, reduce_order="ring")
        st = _call_stats(lambda: ub.ub_gemm_rs_chunked(h, a_t, w.k, w.k, w_t, w.hidden, o_t, w.hidden, cfg, stream),
                         torch, stream)
        row["atomic_gemm_ring_order"] = _stats_row(f, st, MFMA_PEAK_BF16_TFLOPS)
        # the sum fused into the slice-GEMM launch (same bits as the separate reduction)
        for atomic in (False, True):
            cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, False, atomic, fuse_reduce=True)
            st = _call_stats(lambda: ub.ub_gemm_rs_chunked(h, a_t, w.k, w.k, w_t, w.hidden, o_t, w.hidden, cfg, stream),
                             torch, stream)
            row["fused_atomic_gemm" if atomic else "fused_pipeline_3_streams"] = _stats_row(
                f, st, MFMA_PEAK_BF16_TFLOPS)
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

    # GQA bulk sweep on one capacity-32768 buffer, never reallocated
    w = wl.gqa_bulk()
    ra, rw, _ = w.seeds()
    log("secondary gqa_bulk_ag")
    ub_bytes, _ = ub.ub_required_bytes(w.capacity, w.hidden, w.tp)
    ub_t = torch.from_numpy(wl.activations(w, w.capacity, ra).view(np.int16).ravel()).to(dev)
    w_t = torch.from_numpy(wl.weights(w, rw).view(np.int16)).to(dev)
    c_t = torch.empty((w.capacity, w.n_cols), dtype=torch.int16, device=dev)
    h = ub.ub_init(w.capacity, w.hidden, w.tp, ub.UB_DTYPE_BF16, ub_t, ub_bytes)
    res = {}
    for atomic in (True, False):
        cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, False, atomic)
        tot_f = tot_ms = 0.0
        pts = []
        for T in wl.gqa_tokens():
            ub.ub_set_active_shape(h, (T, w.hidden))
            ms, best, _ = _call_stats(lambda: ub.ub_gemm_ag_chunked(h, w_t, w.n_cols, w.n_cols, c_t, w.n_cols, cfg, stream),
                                      torch, stream)
            f = 2.0 * T * w.hidden * w.n_cols
            if T != 32768:
                tot_f += f
                tot_ms += ms
            pts.append((T, round(f / ms / 1e9, 1), round(f / best / 1e9, 1)))
        res["atomic_gemm" if atomic else "host_loop"] = {
            "tflops_sweep": round(tot_f / tot_ms / 1e9, 2),
            "pct_peak_sweep": round(100 * tot_f / tot_ms / 1e9 / MFMA_PEAK_BF16_TFLOPS, 2),
            "points_T_tflops_median_best": pts}
    res["note"] = "per point the median (and best) of 20 calls timed one by one; the sweep is sum FLOPs / sum medians"
    out["gqa_bulk_ag"] = res
    ub.ub_destroy(h)
    return out


def arrival(ub, wl, torch, np, dev):
    """Arrival stand-in on the QKV workload: the 7 non-local ring chunks are copied into the
    UserBuffer on a copy stream while the 8 chunk GEMMs (host loop, 3 streams) wait on their
    own chunk's event, or (modes *_device_loop) while the one device-side chunk loop's tiles
    wait on per-chunk flags written after each copy.  Sources: pinned host memory (SDMA
    over PCIe, about one xGMI link's rate), device memory by SDMA, device memory by the
    runtime's copy kernel (host loop only).  Reports the
    GEMMs alone, the deliveries alone, both overlapped, the fraction of the delivery time
    hidden behind the GEMMs, the overlap as a fraction of the shorter of the two, the time
    the call runs past the deliveries alone, and max(GEMMs, deliveries) / overlapped (1.0
    when the shorter side is wholly hidden; the last chunk's GEMM can only follow its copy,
    so the bound is a little below 1)."""
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


def cpu_baseline(q, min_seconds):
    """The oracle as it stands, timed on the host cores over the same microbatches (whole
    microbatches, in order, repeating passes until at least `min_seconds` of work).  Every
    fourth microbatch of the first pass is also run on the GPU (outside the oracle's timing)
    and compared with the oracle's output: the bit-equal fraction and the largest error as
    a fraction of the gate 4e-3 * |a_row| * |w_col|."""
    import numpy as np

    from oracle import bf16 as ob
    from oracle import gemm as og
    from oracle import manager as om
    from oracle import plan as op

    ub, torch = q.ub, q.torch
    gpu_cfg = q.cfg(atomic=True)
    w_cols = np.linalg.norm(ob.decode(q.w_host), axis=0)
    parity = {"microbatches": 0, "elements": 0, "bit_equal": 0, "max_err_over_gate": 0.0}

    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = sum(i.get("num_threads", 0) for i in libs)
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
                         for i in libs) or "none found"
    except Exception:  # threadpoolctl missing: report the core count
        threads = os.cpu_count()
    w = q.w
    model = om.UserBufferModel(w.capacity, w.hidden, w.tp)
    cfg = op.OverlapCfg(method=w.method, num_splits=w.num_splits,
                        num_max_streams=w.num_max_streams, aggregate=w.aggregate, atomic_gemm=True)
    c = np.empty((w.capacity, w.n_cols), np.uint16)
    flops = elapsed = 0.0
    done = 0
    while elapsed < min_seconds:
        for T in q.Ts:
            model.set_active_shape((T, w.hidden))
            model.fill_active(q.a_host[:T])
            t0 = time.perf_counter()
            og.ag_chunked(model, q.w_host, w.n_cols, w.n_cols, c, w.n_cols, cfg)
            elapsed += time.perf_counter() - t0
            flops += 2.0 * T * w.hidden * w.n_cols
            if done < len(q.Ts) and done % 4 == 0:  # parity of this microbatch, untimed
                ub.ub_set_active_shape(q.h, (T, w.hidden))
                ub.ub_gemm_ag_chunked(q.h, q.w_t, w.n_cols, w.n_cols, q.c_t, w.n_cols, gpu_cfg, q.stream)
                torch.cuda.synchronize()
                g = q.c_t[:T].cpu().numpy().view(np.uint16)
                err = np.abs(ob.decode(g) - ob.decode(c[:T]))
                gate = 4e-3 * np.outer(np.linalg.norm(ob.decode(q.a_host[:T]), axis=1), w_cols)
                parity["microbatches"] += 1
                parity["elements"] += int(g.size)
                parity["bit_equal"] += int(np.sum(g == c[:T]))
                parity["max_err_over_gate"] = max(parity["max_err_over_gate"], float(np.max(err / gate)))
            done += 1
            if elapsed >= min_seconds and done >= len(q.Ts):
                break
        log(f"cpu oracle: {done} microbatches, {elapsed:.1f} s")
    return {"value": round(flops / elapsed / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} qkv microbatches ({done / len(q.Ts):.2f} passes over the 32 of one "
                      f"step), numpy fp64 chunked GEMM + bf16 RNE, {elapsed:.1f} s",
            "host_cpus": os.cpu_count(), "blas": blas,
            "parity": {"microbatches": parity["microbatches"], "elements": parity["elements"],
                       "bit_equal_fraction": round(parity["bit_equal"] / max(1, parity["elements"]), 5),
                       "max_err_over_gate": round(parity["max_err_over_gate"], 5),
                       "note": "device-side chunk loop vs the oracle on every 4th microbatch of one step"}}


if __name__ == "__main__":
    main()
