"""GPU tests of the K-segmented rows of the all-gather-side GEMM (ub_register_scratch).

Rows from seg_row on are summed in nseg K segments, ((P_0 + P_1) + ...) in fp32.  With a
registered scratch the segments run as separate workgroups (split-K) that meet through fp32
partial tiles and per-tile counters; without one, a single workgroup per tile folds the same
segments in the same order.  Checked here: bit-exact against the oracle on integer inputs
(every order of fp32 sums of such products is exact), split == fold == host loop == arrival
bit for bit on random inputs, within the oracle tolerance, the counters back at zero, the
K tail, arrival timeouts inside split tiles, and the automatic choice at the GQA sizes."""

import numpy as np
import pytest
import torch

from chunked_tp_overlap_amd import workloads as wl
from oracle import gemm as og
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MiB = 1 << 20


@pytest.fixture(scope="module")
def ub():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import chunked_tp_overlap_amd.ub as m
    return m


def _scratch(ub, h, nbytes=64 * MiB + 256 * 1024):
    t = torch.zeros(nbytes // 2, dtype=torch.int16, device="cuda")
    ub.ub_register_scratch(h, t, nbytes)
    return t


def _counters_zero(ub, t):
    torch.cuda.synchronize()
    return bool((t[: ub.UB_SCRATCH_COUNTER_BYTES // 2] == 0).all().item())


def _force(ub, h, nseg, seg_row=0):
    ub.ub_debug_set(h, "nseg", nseg)
    ub.ub_debug_set(h, "seg_row", seg_row)


def _seg_tile(ub, h, tile):
    m, n = map(int, tile.split("x"))
    ub.ub_debug_set(h, "seg_tile_m", m)
    ub.ub_debug_set(h, "seg_tile_n", n)


def _run(ub, reg, w_t, n, cfg):
    c = gu.canary((reg.capacity + 4, n))
    ub.ub_gemm_ag_chunked(reg.h, w_t, n, n, c, n, cfg)
    torch.cuda.synchronize()
    ch = gu.host(c)
    assert np.all(ch[reg.capacity:] == gu.CANARY)
    return ch


SCHEDULES = (dict(method="bulk", num_splits=1, atomic_gemm=True),       # device-side loop
             dict(method="pipeline", num_splits=5, atomic_gemm=True),
             dict(method="ring_exchange", num_splits=8),                # host loop, 3 streams
             dict(method="pipeline", num_splits=3, num_max_streams=1))


@pytest.mark.parametrize("H,nseg,seg_row", [
    (2048, 2, 0), (2048, 3, 256), (2048, 8, 500), (1000, 6, 0), (1000, 32, 128), (72, 8, 0)])
def test_integer_inputs_bit_exact(ub, H, nseg, seg_row):
    """Integer inputs: every schedule, split and fold, equals the oracle bit for bit.  H =
    1000 has a K tail (32-deep steps, 31.25 of them) and 6 uneven segments; H = 72 has three
    k-steps, so 8 segments are clamped to 3."""
    rng = np.random.default_rng(H + nseg + seg_row)
    cap, N, T = 2048, 392, 1000   # ragged rows, a partial 128-column tile
    a = wl.integer_bits(rng, (T, H))
    wt = wl.integer_bits(rng, (H, N))
    ref = og.ag_rows(a, wt)
    w_t = gu.dev(wt)
    print(f"[split_k int] H={H} nseg={nseg} seg_row={seg_row}", flush=True)
    reg = gu.Registration(ub, cap, H, 8, workspace=False)
    try:
        reg.set_T(T)
        reg.fill(a)
        _force(ub, reg.h, nseg, seg_row)
        scr = _scratch(ub, reg.h)
        for reduce in (1, 2):
            ub.ub_debug_set(reg.h, "seg_reduce", reduce)
            for tile in gu.BF16_TILES:
                _seg_tile(ub, reg.h, tile)
                for kw in SCHEDULES:
                    c = _run(ub, reg, w_t, N, ub.make_cfg(**kw))
                    assert np.array_equal(c[:T], ref), (reduce, tile, kw)
                    assert np.all(c[T:cap] == gu.CANARY)
                assert _counters_zero(ub, scr)
                # the device-side loop ran split on that tile, with the clamped segment
                # count, or the folding kernel when the tile's partials exceed the scratch
                _run(ub, reg, w_t, N, ub.make_cfg(**SCHEDULES[0]))
                plan = ub.ub_debug_last_plan(reg.h, seg=True)
                ns = min(nseg, (H + 31) // 32)
                bm, bn = map(int, tile.split("x"))
                parts = -(-(T - seg_row) // bm) * -(-N // bn) * ns * bm * bn * 4
                want = (seg_row, ns, reduce, bm, bn) if parts <= 64 * MiB else (seg_row, ns, 0, 128, 128)
                assert plan[5:] == want, plan
        ub.ub_register_scratch(reg.h, None, 0)  # the folding kernel
        for kw in SCHEDULES:
            c = _run(ub, reg, w_t, N, ub.make_cfg(**kw))
            assert np.array_equal(c[:T], ref), ("fold", kw)
    finally:
        reg.close()


def test_split_fold_and_schedules_bit_identical(ub):
    """Random inputs: split-K, the folding kernel, every schedule and the arrival path give
    the same bits for one (seg_row, nseg), within the oracle tolerance; the counters are
    left zero, also after a second, smaller call."""
    rng = np.random.default_rng(77)
    cap, H, N, T = 2048, 4096, 1280, 1496
    a = wl.normal_bits(rng, (T, H))
    wt = wl.normal_bits(rng, (H, N), 0.02)
    w_t = gu.dev(wt)
    ref_o = og.ag_rows(a, wt)
    reg = gu.Registration(ub, cap, H, 8, workspace=False)
    try:
        reg.set_T(T)
        reg.fill(a)
        scr = _scratch(ub, reg.h)
        cases = zip(((4, 0), (3, 640), (8, 1280), (16, 0)), gu.BF16_TILES, (1, 2, 1, 2))
        for (nseg, seg_row), tile, reduce in cases:
            print(f"[split_k rand] nseg={nseg} seg_row={seg_row} tile={tile} reduce={reduce}", flush=True)
            _force(ub, reg.h, nseg, seg_row)
            _seg_tile(ub, reg.h, tile)
            ub.ub_debug_set(reg.h, "seg_reduce", reduce)
            ub.ub_register_scratch(reg.h, scr, scr.numel() * 2)
            ref = _run(ub, reg, w_t, N, ub.make_cfg(**SCHEDULES[0]))[:T]
            gu.check_close(ref, ref_o, a, wt, f"split nseg={nseg}")
            for kw in SCHEDULES[1:]:
                assert np.array_equal(_run(ub, reg, w_t, N, ub.make_cfg(**kw))[:T], ref), kw
            src = gu.dev(a)
            for kw in (dict(method="bulk", num_splits=8, atomic_gemm=True),
                       dict(method="ring_exchange", num_splits=8)):
                c = gu.canary((cap + 4, N))
                ub.ub_gemm_ag_arrival(reg.h, src, w_t, N, N, c, N, ub.make_cfg(**kw))
                torch.cuda.synchronize()
                assert np.array_equal(gu.host(c)[:T], ref), ("arrival", kw)
            assert _counters_zero(ub, scr)
            ub.ub_register_scratch(reg.h, None, 0)  # the folding kernel
            for kw in SCHEDULES:
                assert np.array_equal(_run(ub, reg, w_t, N, ub.make_cfg(**kw))[:T], ref), ("fold", kw)
        # a second, smaller call on the same scratch
        ub.ub_register_scratch(reg.h, scr, scr.numel() * 2)
        _force(ub, reg.h, 6, 0)
        reg.set_T(296)
        c = _run(ub, reg, w_t, N, ub.make_cfg(**SCHEDULES[0]))
        gu.check_close(c[:296], ref_o[:296], a[:296], wt, "split T=296")
        assert np.all(c[296:cap] == gu.CANARY) and _counters_zero(ub, scr)
    finally:
        reg.close()


def test_scratch_too_small_falls_back_to_fold(ub):
    """A launch needing more partial space than registered runs the folding kernel: same
    bits, plan reports split = 0."""
    rng = np.random.default_rng(5)
    cap, H, N, T = 1024, 2048, 1024, 1024
    a = wl.normal_bits(rng, (T, H))
    w_t = gu.dev(wl.normal_bits(rng, (H, N), 0.02))
    reg = gu.Registration(ub, cap, H, 8, workspace=False)
    try:
        reg.set_T(T)
        reg.fill(a)
        _force(ub, reg.h, 8, 0)  # 4 x 4 tiles x 8 segments x 256 KiB = 32 MiB of partials
        scr = _scratch(ub, reg.h)
        cfg = ub.make_cfg(**SCHEDULES[0])
        ref = _run(ub, reg, w_t, N, cfg)
        assert ub.ub_debug_last_plan(reg.h, seg=True)[7] == 2
        ub.ub_register_scratch(reg.h, scr, ub.UB_SCRATCH_COUNTER_BYTES + 16 * MiB)
        assert np.array_equal(_run(ub, reg, w_t, N, cfg), ref)
        assert ub.ub_debug_last_plan(reg.h, seg=True)[5:] == (0, 8, 0, 128, 128)
        with pytest.raises(ub.UBError):
            ub.ub_register_scratch(reg.h, scr, ub.UB_SCRATCH_MIN_BYTES - 2)
        assert _counters_zero(ub, scr)
    finally:
        reg.close()


def test_arrival_timeout_in_split_tiles(ub):
    """No flag is written for the delivered chunks (arrival_drop_flags 1) and the wait
    bound is 2 ms: every segment of the split tiles over those rows runs late, the tiles
    store NaN and count one timeout each; the local chunk's rows are exact and the counters
    are back at zero.  A normal call afterwards is exact again."""
    rng = np.random.default_rng(8)
    cap, H, N, T, tp, rank = 1024, 2048, 256, 1024, 4, 1
    a = wl.integer_bits(rng, (T, H))
    wt = wl.integer_bits(rng, (H, N))
    w_t = gu.dev(wt)
    ref = og.ag_rows(a, wt)
    lo, hi = rank * T // tp, (rank + 1) * T // tp
    reg = gu.Registration(ub, cap, H, tp, workspace=False)
    try:
        reg.set_T(T)
        reg.fill(a)
        scr = _scratch(ub, reg.h)
        _force(ub, reg.h, 4, 0)
        cfg = ub.make_cfg("ring_exchange", rank=rank, atomic_gemm=True)
        # the late rows are whole bands of these tiles: bands x column tiles timeouts when
        # the segments meet in the kernel, one per segment with a separate sum
        for tile, expect, reduce in (("128x128", 6 * 2, 1), ("128x256", 6 * 1, 1), ("256x256", 3 * 1, 1),
                                     ("128x128", 6 * 2 * 4, 2), ("256x256", 3 * 1 * 4, 2)):
            _seg_tile(ub, reg.h, tile)
            ub.ub_debug_set(reg.h, "seg_reduce", reduce)
            before = ub.ub_arrival_timeouts(reg.h)
            ub.ub_debug_set(reg.h, "arrival_wait_us", 2000)
            ub.ub_debug_set(reg.h, "arrival_drop_flags", 1)
            print(f"[split_k arrival] {tile}: flags dropped, 2 ms bound", flush=True)
            c = gu.canary((T, N))
            ub.ub_gemm_ag_arrival(reg.h, gu.dev(a), w_t, N, N, c, N, cfg)
            torch.cuda.synchronize()
            assert ub.ub_debug_last_plan(reg.h, seg=True)[5:] == (0, 4, reduce, *map(int, tile.split("x")))
            ch = gu.host(c)
            assert np.array_equal(ch[lo:hi], ref[lo:hi])
            assert np.all(ch[:lo] == 0x7FC0) and np.all(ch[hi:] == 0x7FC0)
            assert ub.ub_arrival_timeouts(reg.h) - before == expect
            assert _counters_zero(ub, scr)
            ub.ub_debug_set(reg.h, "arrival_drop_flags", 0)
            ub.ub_debug_set(reg.h, "arrival_wait_us", 0)
            print(f"[split_k arrival] {tile}: normal call", flush=True)
            c = gu.canary((T, N))
            ub.ub_gemm_ag_arrival(reg.h, gu.dev(a), w_t, N, N, c, N, cfg)
            torch.cuda.synchronize()
            assert np.array_equal(gu.host(c), ref) and _counters_zero(ub, scr)
    finally:
        reg.close()


@pytest.mark.parametrize("atomic", [True, False])
def test_gqa_automatic_segmentation_sampled(ub, atomic):
    """GQA sizes (hidden 8192, 1280 columns, one 32768-row buffer) with scratch registered:
    sampled rows against the oracle at T where the library segments all rows, only the
    last round's rows, or nothing (T = 8136: one round of the narrow 256x160 tile), and the
    device-side loop's bits equal to the host loop's."""
    w = wl.gqa_bulk()
    ra, rw, _ = w.seeds()
    a_all = wl.activations(w, w.capacity, ra)
    wt = wl.weights(w, rw)
    w_t = gu.dev(wt)
    reg = gu.Registration(ub, w.capacity, w.hidden, w.tp, workspace=False)
    rng = np.random.default_rng(31)
    try:
        reg.fill(a_all)
        scr = _scratch(ub, reg.h)
        c = gu.canary((w.capacity + 4, w.n_cols))
        seen = set()
        for T in (1024, 4072, 8136, 13216, 20328, 32520):
            reg.set_T(T)
            outs = []
            for at in (atomic, not atomic):
                cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, w.aggregate, at)
                c.fill_(gu.CANARY)
                ub.ub_gemm_ag_chunked(reg.h, w_t, w.n_cols, w.n_cols, c, w.n_cols, cfg)
                torch.cuda.synchronize()
                outs.append(gu.host(c))
                if at:
                    plan = ub.ub_debug_last_plan(reg.h, seg=True)
                    seen.add("all" if plan[6] > 1 and plan[5] == 0 else "tail" if plan[6] > 1 else "none")
                    if plan[1] in (192, 160):
                        seen.add("narrow")
            print(f"[gqa split_k] T={T} atomic={atomic} plan={plan}", flush=True)
            ch = outs[0]
            assert np.array_equal(ch[:T], outs[1][:T])
            rows = np.array(sorted(set(rng.integers(0, T, 40).tolist()) | {0, T - 1}))
            gu.check_close(ch[rows], og.ag_rows(a_all[rows], wt), a_all[rows], wt, f"gqa T={T}")
            assert np.all(ch[T:] == gu.CANARY)
        assert _counters_zero(ub, scr)
        assert {"all", "tail", "narrow"} <= seen, seen
    finally:
        reg.close()
