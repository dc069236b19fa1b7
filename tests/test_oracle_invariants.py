"""The invariants the capacity/active-shape method promises, checked on the oracle.

[TE#3564], "Implementation approach in the prototype": views and offsets come from the
active T; the active data is a prefix; nothing is reallocated.  [TE#1344]: chunking and
stream count are scheduling options.  Hence: chunked == unchunked, results independent of
capacity and of the schedule, no byte outside the active region touched, every row
written once, shards concatenate to the full reduce.  Also a planted-mistake test: the
v2.11 behaviour the feature request describes (views from the registered size) must be
caught.
"""

import dataclasses

import numpy as np
import pytest

from chunked_tp_overlap_amd import workloads as wl
from oracle import gemm, manager, plan

CAN = manager.CANARY


def _ag(capacity, hidden, tp, a_bits, w_bits, cfg):
    T = a_bits.shape[0]
    m = manager.UserBufferModel(capacity, hidden, tp)
    assert m.set_active_shape((T, hidden)) == manager.OK
    m.fill_active(a_bits)
    ub_before = m.ub.copy()
    n = w_bits.shape[1]
    c = np.full((capacity + 3, n), CAN, np.uint16)
    st, written = gemm.ag_chunked(m, w_bits, n, n, c, n, cfg)
    assert st == manager.OK
    assert np.array_equal(m.ub, ub_before)  # AG only reads the buffer
    assert np.all(c[T:] == CAN)             # no row at or beyond T written
    assert np.all(written == 1)             # each active row exactly once
    return c[:T]


def _rs(capacity, hidden, tp, a_bits, w_bits, cfg):
    T, k = a_bits.shape
    m = manager.UserBufferModel(capacity, hidden, tp)
    assert m.set_active_shape((T, hidden)) == manager.OK
    out = np.full((capacity + 2, hidden), CAN, np.uint16)
    st, written = gemm.rs_chunked(m, a_bits, k, k, w_bits, hidden, out, hidden, cfg)
    assert st == manager.OK
    assert np.all(out[T:] == CAN)
    assert np.all(m.ws[tp * T * hidden:] == CAN)  # workspace tail beyond tp*T*H untouched
    assert not np.any(m.ws[: tp * T * hidden] == CAN)
    assert np.all(written == 1)
    return out[:T], m


@pytest.fixture(scope="module")
def ag_data():
    rng = np.random.default_rng(21)
    T, H, N = 296, 256, 136  # T = 8 * 37: not a multiple of any chunk count used below
    return wl.normal_bits(rng, (T, H)), wl.normal_bits(rng, (H, N), 0.02)


@pytest.fixture(scope="module")
def rs_data():
    rng = np.random.default_rng(22)
    T, K, H = 232, 512, 96
    return wl.normal_bits(rng, (T, K)), wl.normal_bits(rng, (K, H), 0.02)


def test_ag_chunked_equals_unchunked_and_schedule_free(ag_data):
    a, w = ag_data
    ref = _ag(512, 256, 8, a, w, plan.OverlapCfg(method="bulk", num_splits=1))
    for method in plan.METHODS:
        for ns in (1, 2, 3, 5, 8, 13):
            for nms in (1, 2, 3):
                for agg in (False, True):
                    for rank in (0, 3, 7):
                        cfg = plan.OverlapCfg(method=method, num_splits=ns, num_max_streams=nms,
                                              aggregate=agg, rank=rank)
                        got = _ag(512, 256, 8, a, w, cfg)
                        assert np.array_equal(got, ref), cfg


def test_ag_independent_of_capacity(ag_data):
    a, w = ag_data
    T = a.shape[0]
    cfg = plan.OverlapCfg(num_splits=8)
    ref = _ag(T, 256, 8, a, w, cfg)
    for cap in (T + 8, 512, 1024, 4096):
        assert np.array_equal(_ag(cap, 256, 8, a, w, cfg), ref), cap


def test_rs_schedule_free_and_capacity_free(rs_data):
    a, w = rs_data
    tp = 4
    ref, _ = _rs(232, 96, tp, a, w, plan.OverlapCfg(method="pipeline", num_splits=1))
    for method in plan.METHODS:
        for ns in (1, 2, 4, 7):
            for cap in (232, 512):
                cfg = plan.OverlapCfg(method=method, num_splits=ns, rank=1)
                got, _ = _rs(cap, 96, tp, a, w, cfg)
                assert np.array_equal(got, ref), (cfg, cap)


def test_rs_shards_concatenate_to_full_reduce(rs_data):
    a, w = rs_data
    tp = 8
    T = a.shape[0]
    full, _ = _rs(512, 96, tp, a, w, plan.OverlapCfg(method="pipeline", num_splits=3))
    sh = gemm.shards(full, T, 96, tp)
    assert len(sh) == tp and all(s.shape == (T // tp, 96) for s in sh)
    assert np.array_equal(np.concatenate(sh), full)
    # each shard is what the reduce of just that shard's rows produces
    for r in range(tp):
        rows = slice(r * T // tp, (r + 1) * T // tp)
        out_r, _ = gemm.rs_rows(a[rows], w, tp)
        assert np.array_equal(out_r, sh[r]), r


def test_rs_partials_land_in_packed_prefix(rs_data):
    """Partial slot s of the active T occupies workspace rows [s*T, (s+1)*T)."""
    a, w = rs_data
    tp, T, H = 4, a.shape[0], 96
    _, m = _rs(512, H, tp, a, w, plan.OverlapCfg(method="ring_exchange", num_splits=4))
    _, parts = gemm.rs_rows(a, w, tp)
    for s in range(tp):
        assert np.array_equal(m.ws[s * T * H:(s + 1) * T * H].reshape(T, H), parts[s])


def test_ag_sample_rows_match_chunked(ag_data):
    a, w = ag_data
    full = _ag(512, 256, 8, a, w, plan.OverlapCfg(num_splits=8))
    rows = np.array([0, 1, 36, 37, 150, 295])
    assert np.array_equal(gemm.ag_rows(a[rows], w), full[rows])


def test_shape_change_reuses_the_same_buffer(ag_data):
    """Many active shapes over one registration: each result equals a fresh run."""
    a, w = ag_data
    m = manager.UserBufferModel(512, 256, 8)
    ub_id = id(m.ub)
    n = w.shape[1]
    for T in (8, 296, 64, 200, 16):
        assert m.set_active_shape((T, 256)) == manager.OK
        m.fill_active(a[:T])
        c = np.full((512, n), CAN, np.uint16)
        st, _ = gemm.ag_chunked(m, w, n, n, c, n, plan.OverlapCfg(num_splits=8))
        assert st == manager.OK and id(m.ub) == ub_id and m.ub.size == 512 * 256
        assert np.array_equal(c[:T], gemm.ag_rows(a[:T], w))
        assert np.all(c[T:] == CAN)


def test_planted_capacity_offsets_are_caught(monkeypatch):
    """Plant the registered-size mistake ([TE#3564], "Problem": views and counts taken
    from the registered buffer size) into the oracle's chunk plan, on the CPU, and show
    the checks catch it.  With capacity 512, active T = 128 and 4 chunks, the planted
    plan reads rows [128, 512) -- canary -- and writes output rows past T; a second
    variant keeps the rows but reads each chunk at its capacity-based offset."""
    w = wl.tiny_ag()
    ra, rw, _ = w.seeds()
    a = wl.activations(w, 128, ra)
    wt = wl.weights(w, rw)
    cfg = plan.OverlapCfg(method="bulk", num_splits=4)
    good = _ag(w.capacity, w.hidden, w.tp, a, wt, cfg)

    real_build = plan.build
    monkeypatch.setattr(plan, "build", lambda T, tp, c, op, stream_limit=None:
                        real_build(w.capacity, tp, c, op, stream_limit))
    with pytest.raises(AssertionError):
        _ag(w.capacity, w.hidden, w.tp, a, wt, cfg)

    monkeypatch.undo()
    # second planted variant: rows planned from T, but the read offset of a chunk taken
    # from the registered size (chunk c at c * capacity / n rows)
    monkeypatch.setattr(manager.UserBufferModel, "row_offset_elems",
                        lambda self, row0: (row0 * self.capacity // self.T) * self.hidden)
    m = manager.UserBufferModel(w.capacity, w.hidden, w.tp)
    m.set_active_shape((128, w.hidden))
    m.fill_active(a)
    n = wt.shape[1]
    c = np.full((w.capacity, n), CAN, np.uint16)
    gemm.ag_chunked(m, wt, n, n, c, n, cfg)
    assert np.array_equal(c[:32], good[:32])      # chunk 0 starts at row 0 either way
    assert not np.array_equal(c[32:128], good[32:128])  # the others read canary rows


def test_capacity_offset_of_a_chunk_points_at_canary():
    """Reading chunk 1 at ``1 * (capacity / n) * H`` instead of ``floor(T / n) * H``
    after shrinking T lands in the canary-filled tail of the buffer."""
    w = wl.tiny_ag()
    ra, _, _ = w.seeds()
    a = wl.activations(w, 128, ra)
    m = manager.UserBufferModel(w.capacity, w.hidden, w.tp)
    m.set_active_shape((128, w.hidden))
    m.fill_active(a)
    H, n = w.hidden, 2
    bad_off = 1 * (w.capacity // n) * H
    good_off = m.row_offset_elems(128 // n)
    assert bad_off != good_off
    assert np.all(m.ub[bad_off: bad_off + 64 * H] == CAN)
    assert not np.any(m.ub[good_off: good_off + 64 * H] == CAN)
