"""GPU tests of the arrival stand-in (ub_gemm_ag_arrival, ub_deliver_chunks): the non-local
chunks are copied into the UserBuffer on a copy stream while the GEMM units that need them
wait on per-chunk events (host loop) or, in the device-side chunk loop, the tiles wait on
per-chunk flags that the copy stream writes after each copy.  Results must be bit-identical to the all-gather GEMM over a
complete buffer, the local chunk's rows of the source are never read, and nothing beyond
the active prefix is touched."""

import numpy as np
import pytest
import torch

from chunked_tp_overlap_amd import workloads as wl
from oracle import gemm as og
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ub():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import chunked_tp_overlap_amd.ub as m
    return m


def _local_rows(method, rank, T, tp):
    if method != "ring_exchange":
        return None
    return (rank * T // tp, (rank + 1) * T // tp)


def _pinned(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).pin_memory()


def _case(ub, reg, a, w_t, N, cfg_kw, ref, T, tp, host_src=False):
    """UB: canary except the local chunk; src: every row, local rows replaced by canary
    (device memory, or pinned host memory when host_src)."""
    H = reg.hidden
    loc = _local_rows(cfg_kw["method"], cfg_kw.get("rank", 0), T, tp)
    reg.ub_t.fill_(gu.CANARY)
    src_h = a.copy()
    if loc:
        reg.ub_t[loc[0] * H: loc[1] * H].copy_(gu.dev(a[loc[0]:loc[1]]).reshape(-1))
        src_h[loc[0]:loc[1]] = gu.CANARY
    src = _pinned(src_h) if host_src else gu.dev(src_h)
    c = gu.canary((reg.capacity + 4, N))
    ub.ub_gemm_ag_arrival(reg.h, src, w_t, N, N, c, N, ub.make_cfg(**cfg_kw))
    torch.cuda.synchronize()
    ch = gu.host(c)
    assert np.array_equal(ch[:T], ref), cfg_kw
    assert np.all(ch[T:] == gu.CANARY)
    ubh = gu.host(reg.ub_t)
    assert np.array_equal(ubh[: T * H].reshape(T, H), a), cfg_kw  # prefix complete
    assert np.all(ubh[T * H:] == gu.CANARY)


def test_arrival_bit_identical_to_complete_buffer(ub):
    rng = np.random.default_rng(51)
    cap, H, N, T, tp = 1024, 512, 264, 600, 8
    a = wl.normal_bits(rng, (T, H))
    w_t = gu.dev(wl.normal_bits(rng, (H, N), 0.02))
    reg = gu.Registration(ub, cap, H, tp, workspace=False, pad_rows=8)
    try:
        reg.set_T(T)
        reg.fill(a)
        c = gu.canary((T, N))
        ub.ub_gemm_ag_chunked(reg.h, w_t, N, N, c, N, ub.make_cfg("bulk", 1))
        torch.cuda.synchronize()
        ref = gu.host(c)
        for kw in (dict(method="ring_exchange", rank=0), dict(method="ring_exchange", rank=5),
                   dict(method="ring_exchange", rank=3, aggregate=True),
                   dict(method="ring_exchange", rank=7, num_max_streams=1),
                   dict(method="pipeline", num_splits=5), dict(method="bulk", num_splits=3, aggregate=True)):
            for use_ce in (True, False):
                print(f"[arrival] {kw} use_ce={use_ce}", flush=True)
                _case(ub, reg, a, w_t, N, dict(kw, use_ce=use_ce), ref, T, tp)
            print(f"[arrival] {kw} host source", flush=True)
            _case(ub, reg, a, w_t, N, kw, ref, T, tp, host_src=True)
            # the device-side chunk loop gated by per-chunk flags: SDMA and host sources
            print(f"[arrival] {kw} atomic_gemm, SDMA", flush=True)
            _case(ub, reg, a, w_t, N, dict(kw, atomic_gemm=True, use_ce=True), ref, T, tp)
            print(f"[arrival] {kw} atomic_gemm, host source", flush=True)
            _case(ub, reg, a, w_t, N, dict(kw, atomic_gemm=True), ref, T, tp, host_src=True)
        assert ub.ub_arrival_timeouts(reg.h) == 0
        with pytest.raises(ub.UBError) as e:  # copy-kernel deliveries cannot gate the loop
            ub.ub_gemm_ag_arrival(reg.h, gu.dev(a), w_t, N, N, gu.canary((T, N)), N,
                                  ub.make_cfg("pipeline", 4, atomic_gemm=True, use_ce=False))
        assert e.value.name == "UB_ERR_UNSUPPORTED"
    finally:
        reg.close()


def test_arrival_device_loop_flag_slots(ub):
    """Flag slots: two handles gate at once, and 70 handles in a row (more than the 64
    slots) each take and return one."""
    rng = np.random.default_rng(54)
    cap, H, N, T, tp = 256, 128, 64, 256, 4
    a = wl.normal_bits(rng, (T, H))
    w_t = gu.dev(wl.normal_bits(rng, (H, N), 0.02))
    src = gu.dev(a)
    ref_reg = gu.Registration(ub, cap, H, tp, workspace=False)
    try:
        ref_reg.set_T(T)
        ref_reg.fill(a)
        ref = gu.canary((T, N))
        ub.ub_gemm_ag_chunked(ref_reg.h, w_t, N, N, ref, N, ub.make_cfg("bulk", 1))
        torch.cuda.synchronize()
        ref = gu.host(ref)
    finally:
        ref_reg.close()
    regs = [gu.Registration(ub, cap, H, tp, workspace=False) for _ in range(2)]
    try:
        outs = []
        for i, r in enumerate(regs):  # both calls in flight on the null stream's order
            r.set_T(T)
            r.ub_t.fill_(gu.CANARY)
            c = gu.canary((T, N))
            ub.ub_gemm_ag_arrival(r.h, src, w_t, N, N, c, N,
                                  ub.make_cfg("pipeline", 4, atomic_gemm=True))
            outs.append(c)
        torch.cuda.synchronize()
        for c in outs:
            assert np.array_equal(gu.host(c), ref)
        assert all(ub.ub_arrival_timeouts(r.h) == 0 for r in regs)
    finally:
        for r in regs:
            r.close()
    for i in range(70):
        r = gu.Registration(ub, cap, H, tp, workspace=False)
        try:
            r.set_T(T)
            c = gu.canary((T, N))
            ub.ub_gemm_ag_arrival(r.h, src, w_t, N, N, c, N, ub.make_cfg("ring_exchange", rank=i % tp,
                                                                           atomic_gemm=True))
            torch.cuda.synchronize()
            lo, hi = (i % tp) * T // tp, (i % tp + 1) * T // tp
            got = gu.host(c)
            # the local chunk was never written (canary), so only the delivered rows compare
            assert np.array_equal(np.delete(got, np.s_[lo:hi], axis=0), np.delete(ref, np.s_[lo:hi], axis=0)), i
            assert ub.ub_arrival_timeouts(r.h) == 0
        finally:
            r.close()


def test_deliver_chunks_alone(ub):
    rng = np.random.default_rng(52)
    cap, H, T, tp, rank = 512, 256, 296, 8, 2
    a = wl.normal_bits(rng, (T, H))
    reg = gu.Registration(ub, cap, H, tp, workspace=False, pad_rows=8)
    try:
        reg.set_T(T)
        for use_ce, src in ((True, gu.dev(a)), (False, gu.dev(a)), (True, _pinned(a))):
            reg.ub_t.fill_(gu.CANARY)
            ub.ub_deliver_chunks(reg.h, src, ub.make_cfg("ring_exchange", rank=rank, use_ce=use_ce))
            torch.cuda.synchronize()
            got = gu.host(reg.ub_t)[: T * H].reshape(T, H)
            lo, hi = rank * T // tp, (rank + 1) * T // tp
            assert np.array_equal(got[:lo], a[:lo]) and np.array_equal(got[hi:], a[hi:])
            assert np.all(got[lo:hi] == gu.CANARY)  # the local chunk is not delivered
            assert np.all(gu.host(reg.ub_t)[T * H:] == gu.CANARY)
    finally:
        reg.close()


def test_arrival_ordered_after_caller_stream_work(ub):
    """The local shard is written on the caller's stream right before the call (no host
    synchronisation): the copies and GEMMs must see it."""
    rng = np.random.default_rng(53)
    cap, H, N, T, tp, rank = 512, 256, 128, 256, 4, 1
    a = wl.normal_bits(rng, (T, H))
    w = wl.normal_bits(rng, (H, N), 0.02)
    reg = gu.Registration(ub, cap, H, tp, workspace=False)
    s = torch.cuda.Stream()
    try:
        reg.set_T(T)
        lo, hi = rank * T // tp, (rank + 1) * T // tp
        src_h = a.copy()
        src_h[lo:hi] = gu.CANARY
        src, loc, w_t = gu.dev(src_h), gu.dev(a[lo:hi]), gu.dev(w)
        c = gu.canary((T, N))
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            reg.ub_t.fill_(gu.CANARY)
            torch.cuda._sleep(2_000_000)  # keep the stream busy before the writes land
            ub.ub_copy_in(reg.h, loc, hi - lo, lo, s)
            ub.ub_gemm_ag_arrival(reg.h, src, w_t, N, N, c, N, ub.make_cfg("ring_exchange", rank=rank), s)
        torch.cuda.synchronize()
        gu.check_close(gu.host(c), og.ag_rows(a, w, N), a, w, "arrival stream order")
    finally:
        reg.close()


def test_arrival_qkv_full_size(ub):
    """The QKV workload at T = 8192 (capacity 8192, hidden 4096, W [4096, 1536], ring of
    8): bit-identical to the GEMM over the complete buffer, sampled rows vs the oracle."""
    w = wl.qkv()
    ra, rw, _ = w.seeds()
    T = w.capacity
    a = wl.activations(w, T, ra)
    wt = wl.weights(w, rw)
    N, H, tp = w.n_cols, w.hidden, w.tp
    w_t = gu.dev(wt)
    reg = gu.Registration(ub, w.capacity, H, tp, workspace=False, pad_rows=8)
    try:
        reg.set_T(T)
        reg.fill(a)
        c = gu.canary((T, N))
        ub.ub_gemm_ag_chunked(reg.h, w_t, N, N, c, N, ub.make_cfg("ring_exchange", atomic_gemm=True))
        torch.cuda.synchronize()
        ref = gu.host(c)
        for use_ce, host_src, atomic in ((True, False, False), (False, False, False), (True, True, False),
                                         (True, False, True), (True, True, True)):
            print(f"[arrival qkv] use_ce={use_ce} host_src={host_src} atomic={atomic}", flush=True)
            _case(ub, reg, a, w_t, N, dict(method="ring_exchange", rank=3, use_ce=use_ce,
                                           atomic_gemm=atomic), ref, T, tp, host_src=host_src)
        assert ub.ub_arrival_timeouts(reg.h) == 0
        rows = np.array(sorted({0, 1, T // 2, T - 1} | {r * T // tp for r in range(tp)}))
        gu.check_close(ref[rows], og.ag_rows(a[rows], wt, N), a[rows], wt, "arrival qkv rows")
    finally:
        reg.close()


def test_arrival_device_loop_wait_bound(ub):
    """The failure path of the device-side loop's wait, forced from the host through the
    handle's debug settings: no flag is written for the delivered chunks
    (arrival_drop_flags 1) and the bound is 2 ms (arrival_wait_us), so the tiles that need
    those chunks give up, count one timeout each, store NaN over their output, and end: the
    call returns and nothing hangs.  The tiles of the local chunk, whose flag is written,
    are still right.  A normal call afterwards is bit-identical to the complete-buffer GEMM
    and adds no timeout."""
    rng = np.random.default_rng(55)
    cap, H, N, T, tp, rank = 1024, 512, 264, 1024, 4, 1
    a = wl.normal_bits(rng, (T, H))
    w_t = gu.dev(wl.normal_bits(rng, (H, N), 0.02))
    reg = gu.Registration(ub, cap, H, tp, workspace=False, pad_rows=8)
    gu.force_tile(ub, reg.h, "256x256")  # the local chunk is exactly one tile row
    try:
        reg.set_T(T)
        reg.fill(a)
        ref = gu.canary((T, N))
        ub.ub_gemm_ag_chunked(reg.h, w_t, N, N, ref, N, ub.make_cfg("bulk", 1))
        torch.cuda.synchronize()
        ref = gu.host(ref)
        lo, hi = rank * T // tp, (rank + 1) * T // tp
        cfg = ub.make_cfg("ring_exchange", rank=rank, atomic_gemm=True)
        before = ub.ub_arrival_timeouts(reg.h)
        ub.ub_debug_set(reg.h, "arrival_wait_us", 2000)
        ub.ub_debug_set(reg.h, "arrival_drop_flags", 1)
        print("[arrival wait bound] flags dropped, 2 ms bound", flush=True)
        c = gu.canary((T, N))
        ub.ub_gemm_ag_arrival(reg.h, gu.dev(a), w_t, N, N, c, N, cfg)
        torch.cuda.synchronize()
        after = ub.ub_arrival_timeouts(reg.h)
        # 3 bands of 256 rows whose chunks never came, 2 column tiles each
        assert after - before == 3 * 2
        got = gu.host(c)
        assert np.array_equal(got[lo:hi], ref[lo:hi])
        late = np.concatenate([got[:lo], got[hi:]])
        assert np.all(late == 0x7FC0)
        ub.ub_debug_set(reg.h, "arrival_wait_us", 0)
        ub.ub_debug_set(reg.h, "arrival_drop_flags", 0)
        print("[arrival wait bound] normal call", flush=True)
        _case(ub, reg, a, w_t, N, dict(method="ring_exchange", rank=rank, atomic_gemm=True), ref, T, tp)
        assert ub.ub_arrival_timeouts(reg.h) == after
        # destroying the handle clears its slot's count: a new handle (which takes the
        # lowest free slot, the one just released) starts from zero
        reg.close()
        reg = gu.Registration(ub, cap, H, tp, workspace=False, pad_rows=8)
        reg.set_T(T)
        print("[arrival wait bound] next handle", flush=True)
        _case(ub, reg, a, w_t, N, dict(method="ring_exchange", rank=rank, atomic_gemm=True), ref, T, tp)
        assert ub.ub_arrival_timeouts(reg.h) == 0
    finally:
        reg.close()


def test_arrival_device_loop_with_cut(ub):
    """The device-side loop gated on arrivals when its tile plan is cut in two launches
    (13216 rows x 1280 columns; a cut forced after 51 bands of 256 rows, the last 160 rows
    as 128 x 128 tiles): both launches wait on the flags of the chunks they read, no wait
    runs into its bound, and the output equals the ungated GEMM over the complete buffer
    bit for bit.  The handle's timeout count starts at zero even when its flag slot was
    used (and timed out on purpose) by a handle destroyed before it."""
    rng = np.random.default_rng(57)
    cap, H, N, T, tp = 13312, 256, 1280, 13216, 8
    a = wl.normal_bits(rng, (T, H))
    w_t = gu.dev(wl.normal_bits(rng, (H, N), 0.02))
    reg = gu.Registration(ub, cap, H, tp, workspace=False, pad_rows=8)
    try:
        reg.set_T(T)
        reg.fill(a)
        c = gu.canary((T, N))
        ub.ub_gemm_ag_chunked(reg.h, w_t, N, N, c, N, ub.make_cfg("bulk", 1, 1))
        torch.cuda.synchronize()
        ref = gu.host(c)
        gu.force_tile(ub, reg.h, "256x256")
        ub.ub_debug_set(reg.h, "cut_row", 51 * 256)
        for rank, host_src in ((0, False), (5, False), (3, True)):
            print(f"[arrival cut] rank={rank} host_src={host_src}", flush=True)
            _case(ub, reg, a, w_t, N, dict(method="ring_exchange", rank=rank, atomic_gemm=True,
                                          use_ce=True), ref, T, tp, host_src=host_src)
            assert ub.ub_debug_last_plan(reg.h) == (256, 256, 51 * 256, 128, 128)
        assert ub.ub_arrival_timeouts(reg.h) == 0
    finally:
        reg.close()
