#!/usr/bin/env python3
"""Benchmark of the chunked tensor-parallel overlap GEMMs on one MI355X.

Metric: bf16 TFLOP/s of the chunked AG/RS GEMM at the active T, and its fraction of the
dense bf16 MFMA peak.  One step = one pass of the hot path over one batch of the QKV
workload: for each of its 32 THD microbatches, set the active shape [T, 4096] on the one
capacity-8192 UserBuffer and run the chunked all-gather-side GEMM (W [4096, 1536], ring
exchange over tp = 8 chunks, 3 compute streams).  FLOPs are algorithmic: 2 * T * 4096 *
1536 per microbatch, active T only.  Inputs are seeded synthetic draws already resident
in HBM when the timed region starts.

The other workloads (fc1 with aggregate, fc2 reduce-scatter with its reduction, the GQA
bulk sweep) are measured after the timed region and reported under "secondary".
Prints one JSON line.
"""

import argparse
import json
import os
import sys
import time

MFMA_PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense
HBM_PEAK_GBS = 8000.0


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="bound on the CPU-oracle baseline sample (seconds of work)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the work on a single MI355X; "
              f"--gpus {args.gpus} (WORLD_SIZE={world}) is not supported: this build has no "
              "multi-GPU path.", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import chunked_tp_overlap_amd.ub as ub
    from chunked_tp_overlap_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    # ---- the QKV workload -------------------------------------------------------------
    w = wl.qkv()
    ra, rw, rt = w.seeds()
    Ts, packs = wl.qkv_pack_tokens(rt)
    log(f"generating inputs: capacity {w.capacity} x {w.hidden}, W {w.hidden} x {w.n_cols}")
    a_host = wl.activations(w, w.capacity, ra)
    w_host = wl.weights(w, rw)
    ub_bytes, _ = ub.ub_required_bytes(w.capacity, w.hidden, w.tp)
    ub_t = torch.from_numpy(a_host.view(np.int16).ravel()).to(dev)
    w_t = torch.from_numpy(w_host.view(np.int16)).to(dev)
    c_t = torch.empty((w.capacity, w.n_cols), dtype=torch.int16, device=dev)
    h = ub.ub_init(w.capacity, w.hidden, w.tp, ub.UB_DTYPE_BF16, ub_t, ub_bytes)
    cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, w.aggregate)
    stream = torch.cuda.current_stream()
    step_flops = sum(2.0 * T * w.hidden * w.n_cols for T in Ts)

    def step():
        for T in Ts:
            ub.ub_set_active_shape(h, (T, w.hidden))
            ub.ub_gemm_ag_chunked(h, w_t, w.n_cols, w.n_cols, c_t, w.n_cols, cfg, stream)

    log(f"warmup {args.warmup} steps of {len(Ts)} microbatches")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ub.ub_set_kernel_timing(h, True)
    ub.ub_get_kernel_timing(h)  # clear
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gemm_stats, _ = ub.ub_get_kernel_timing(h)
    ub.ub_set_kernel_timing(h, False)
    wall = t1 - t0
    ev_ms = ev0.elapsed_time(ev1)
    tflops = step_flops * args.steps / wall / 1e12
    log(f"timed {args.steps} steps: {wall * 1e3:.2f} ms wall, {ev_ms:.2f} ms events, "
        f"{tflops:.1f} TFLOP/s")

    # per-microbatch times, one launch sequence each, for the T >= 4096 aggregate
    per_mb = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for T in Ts:
        ub.ub_set_active_shape(h, (T, w.hidden))
        ub.ub_gemm_ag_chunked(h, w_t, w.n_cols, w.n_cols, c_t, w.n_cols, cfg, stream)
        reps = 5
        e0.record(stream)
        for _ in range(reps):
            ub.ub_gemm_ag_chunked(h, w_t, w.n_cols, w.n_cols, c_t, w.n_cols, cfg, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        per_mb.append((T, e0.elapsed_time(e1) / reps))
    big = [(T, ms) for T, ms in per_mb if T >= 4096]
    agg_ge4096 = sum(2.0 * T * w.hidden * w.n_cols for T, _ in big) / (sum(ms for _, ms in big) / 1e3) / 1e12

    g_ach = gemm_stats["flops"] / (gemm_stats["total_ms"] / 1e3) / 1e12 if gemm_stats["launches"] else 0.0
    roofline = {
        "bound": "mfma", "kernel": "gemm_bf16 (per-unit chunk GEMM)",
        "achieved": round(g_ach, 2), "peak": MFMA_PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(g_ach / MFMA_PEAK_BF16_TFLOPS, 4), "traffic": None,
        "launches": gemm_stats["launches"],
        "avg_launch_us": round(gemm_stats["total_ms"] * 1e3 / max(1, gemm_stats["launches"]), 3),
        "avg_launch_gflop": round(gemm_stats["flops"] / max(1, gemm_stats["launches"]) / 1e9, 4),
    }

    result = {
        "metric": "bf16 TFLOP/s of chunked AG/RS GEMM at active T; % of MFMA peak",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_mfma_peak": round(100 * tflops / MFMA_PEAK_BF16_TFLOPS, 2),
        "config": {
            "workload": "qkv_ag: column-parallel AG-GEMM over a [8192, 4096] bf16 UserBuffer, "
                        "W [4096, 1536], tp 8, ring exchange (8 chunks), 3 streams, "
                        "32 THD microbatches per step",
            "capacity": w.capacity, "hidden": w.hidden, "n_cols": w.n_cols, "tp": w.tp,
            "method": w.method, "num_splits": w.num_splits, "num_max_streams": w.num_max_streams,
            "microbatches": len(Ts), "T_min": min(Ts), "T_max": max(Ts),
            "T_mean": round(sum(Ts) / len(Ts), 1), "gflop_per_step": round(step_flops / 1e9, 2),
            "seed": w.seed,
        },
        "event_ms_per_step": round(ev_ms / args.steps, 4),
        "tflops_T_ge_4096_per_microbatch_aggregate": round(agg_ge4096, 3),
        "roofline": roofline,
    }

    props = torch.cuda.get_device_properties(0)
    result["device"] = {"name": props.name, "cus": props.multi_processor_count,
                        "gcn_arch": getattr(props, "gcnArchName", "")}

    if not args.no_secondary:
        result["secondary"] = secondary(ub, wl, torch, np, dev, log)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, Ts, a_host, w_host, args.cpu_seconds, log)

    ub.ub_destroy(h)
    print(json.dumps(result), flush=True)


def _time_calls(fn, torch, stream, reps):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def secondary(ub, wl, torch, np, dev, log):
    out = {}
    stream = torch.cuda.current_stream()

    # fc1: aggregate-2x, 16 microbatches
    w = wl.fc1()
    ra, rw, rt = w.seeds()
    Ts = wl.fc1_tokens(rt)
    log("secondary fc1_ag")
    ub_bytes, _ = ub.ub_required_bytes(w.capacity, w.hidden, w.tp)
    ub_t = torch.from_numpy(wl.activations(w, w.capacity, ra).view(np.int16).ravel()).to(dev)
    w_t = torch.from_numpy(wl.weights(w, rw).view(np.int16)).to(dev)
    c_t = torch.empty((w.capacity, w.n_cols), dtype=torch.int16, device=dev)
    h = ub.ub_init(w.capacity, w.hidden, w.tp, ub.UB_DTYPE_BF16, ub_t, ub_bytes)
    cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, w.aggregate)
    tot_f = tot_ms = big_f = big_ms = 0.0
    for T in Ts:
        ub.ub_set_active_shape(h, (T, w.hidden))
        ms = _time_calls(lambda: ub.ub_gemm_ag_chunked(h, w_t, w.n_cols, w.n_cols, c_t, w.n_cols, cfg, stream),
                         torch, stream, 5)
        f = 2.0 * T * w.hidden * w.n_cols
        tot_f += f
        tot_ms += ms
        if T >= 4096:
            big_f += f
            big_ms += ms
    out["fc1_ag"] = {"tflops_all": round(tot_f / tot_ms / 1e9, 2),
                     "tflops_T_ge_4096": round(big_f / big_ms / 1e9, 2) if big_ms else None,
                     "pct_peak_T_ge_4096": round(100 * big_f / big_ms / 1e9 / MFMA_PEAK_BF16_TFLOPS, 2) if big_ms else None,
                     "microbatches": len(Ts)}
    ub.ub_destroy(h)
    del ub_t, w_t, c_t

    # fc2: row-parallel RS GEMM + reduction over the T sweep
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
    cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams)
    rows = []
    for T in wl.FC2_TOKENS:
        ub.ub_set_active_shape(h, (T, w.hidden))
        ms = _time_calls(lambda: ub.ub_gemm_rs_chunked(h, a_t, w.k, w.k, w_t, w.hidden, o_t, w.hidden, cfg, stream),
                         torch, stream, 5)
        f = 2.0 * T * w.k * w.hidden
        rbytes = (w.tp + 1) * T * w.hidden * 2.0
        warm = _time_calls(lambda: ub.ub_reduce_partials(h, o_t, w.hidden, stream), torch, stream, 10)
        # honest: a 768 MB write between reductions evicts the 256 MB MALL
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cold = []
        for _ in range(5):
            flush.fill_(1)
            e0.record(stream)
            ub.ub_reduce_partials(h, o_t, w.hidden, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        cold_ms = sorted(cold)[len(cold) // 2]
        rows.append({"T": T, "tflops": round(f / ms / 1e9, 2),
                     "pct_peak": round(100 * f / ms / 1e9 / MFMA_PEAK_BF16_TFLOPS, 2),
                     "ms": round(ms, 4),
                     "reduce_gbs_warm": round(rbytes / warm / 1e6, 1),
                     "reduce_gbs_flushed": round(rbytes / cold_ms / 1e6, 1),
                     "reduce_pct_hbm_flushed": round(100 * rbytes / cold_ms / 1e6 / HBM_PEAK_GBS, 2)})
    out["fc2_rs"] = rows
    ub.ub_destroy(h)
    del ub_t, ws_t, a_t, w_t, o_t, flush

    # GQA bulk sweep on one capacity-32768 buffer
    w = wl.gqa_bulk()
    ra, rw, _ = w.seeds()
    log("secondary gqa_bulk_ag")
    ub_bytes, _ = ub.ub_required_bytes(w.capacity, w.hidden, w.tp)
    ub_t = torch.from_numpy(wl.activations(w, w.capacity, ra).view(np.int16).ravel()).to(dev)
    w_t = torch.from_numpy(wl.weights(w, rw).view(np.int16)).to(dev)
    c_t = torch.empty((w.capacity, w.n_cols), dtype=torch.int16, device=dev)
    h = ub.ub_init(w.capacity, w.hidden, w.tp, ub.UB_DTYPE_BF16, ub_t, ub_bytes)
    cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams)
    tot_f = tot_ms = 0.0
    pts = []
    for T in wl.gqa_tokens():
        ub.ub_set_active_shape(h, (T, w.hidden))
        ms = _time_calls(lambda: ub.ub_gemm_ag_chunked(h, w_t, w.n_cols, w.n_cols, c_t, w.n_cols, cfg, stream),
                         torch, stream, 3)
        f = 2.0 * T * w.hidden * w.n_cols
        if T != 32768:
            tot_f += f
            tot_ms += ms
        pts.append((T, round(f / ms / 1e9, 1)))
    out["gqa_bulk_ag"] = {"tflops_sweep": round(tot_f / tot_ms / 1e9, 2),
                          "pct_peak_sweep": round(100 * tot_f / tot_ms / 1e9 / MFMA_PEAK_BF16_TFLOPS, 2),
                          "points_T_tflops": pts[::4] + [pts[-1]]}
    ub.ub_destroy(h)
    return out


def cpu_baseline(w, Ts, a_host, w_host, budget_s, log):
    """The oracle as it stands, timed on the host cores over a bounded sample of the
    same microbatches (whole microbatches, in order, until the time budget is used)."""
    import numpy as np

    from oracle import gemm as og
    from oracle import manager as om
    from oracle import plan as op

    try:
        from threadpoolctl import threadpool_info
        threads = sum(i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas")
    except Exception:  # threadpoolctl missing: report the core count
        threads = os.cpu_count()
    model = om.UserBufferModel(w.capacity, w.hidden, w.tp)
    cfg = op.OverlapCfg(method=w.method, num_splits=w.num_splits,
                        num_max_streams=w.num_max_streams, aggregate=w.aggregate)
    c = np.empty((w.capacity, w.n_cols), np.uint16)
    flops = 0.0
    elapsed = 0.0
    done = 0
    for T in Ts:
        model.set_active_shape((T, w.hidden))
        model.fill_active(a_host[:T])
        t0 = time.perf_counter()
        og.ag_chunked(model, w_host, w.n_cols, w.n_cols, c, w.n_cols, cfg)
        elapsed += time.perf_counter() - t0
        flops += 2.0 * T * w.hidden * w.n_cols
        done += 1
        log(f"cpu oracle: {done} microbatches, {elapsed:.1f} s")
        if elapsed >= budget_s:
            break
    return {"value": round(flops / elapsed / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {done} of {len(Ts)} qkv microbatches (T={Ts[:done]}), numpy fp64 "
                      f"chunked GEMM + bf16 RNE, {elapsed:.1f} s",
            "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
