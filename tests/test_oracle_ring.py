"""Pins of the ring-order reduce-scatter of the oracle (reduce_order="ring").

The rule: the partials of shard r travel the ring from rank r+1 to rank r; every hop
adds a bf16 partial to the arriving bf16 value in fp32 and rounds the sum to bf16.
Pinned by hand-worked cases (tests/golden/ring_reduce_hops.txt), by an integer brute
force of the same rule (tests/exact.py), and by the invariants the method promises.
"""

import os

import numpy as np
import pytest

from chunked_tp_overlap_amd import workloads as wl
from oracle import bf16, gemm, manager, plan
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ring_reduce_hops.txt")


def _golden():
    cases = []
    with open(GOLDEN) as f:
        for ln in f:
            ln = ln.split("#")[0].strip()
            if not ln:
                continue
            head, parts, ring, asc = (x.strip() for x in ln.split("|"))
            tp, shard = (int(x) for x in head.split())
            vals = [float(x) for x in parts.split()]
            assert len(vals) == tp
            cases.append((tp, shard, vals, int(ring, 16), int(asc, 16)))
    return cases


@pytest.mark.parametrize("case", _golden())
def test_hand_worked_cases(case):
    tp, shard, vals, ring_bits, asc_bits = case
    parts = [np.array([[v]]) for v in vals]
    assert np.array_equal(bf16.decode(bf16.encode_rne(np.array(vals))), np.array(vals))
    got = gemm.ring_sum(parts, shard, tp, tp)  # T = tp: one row per shard
    assert int(got[0, 0]) == ring_bits, hex(int(got[0, 0]))
    asc = bf16.encode_rne(gemm.exact_sum(parts) + 0.0)
    assert int(asc[0, 0]) == asc_bits


@pytest.mark.parametrize("tp", [2, 3, 4, 8])
def test_ring_sum_equals_integer_brute_force(tp):
    rng = np.random.default_rng(100 + tp)
    T, n = tp * 5, 12
    # partials of mixed magnitudes (nonzero), so hops round at various exponents
    parts_bits = []
    for s in range(tp):
        x = rng.standard_normal((T, n)) * np.exp2(rng.integers(-6, 7, size=(T, n)))
        parts_bits.append(bf16.encode_rne(np.where(x == 0, 1.0, x)))
    got = gemm.ring_sum([bf16.decode(p) for p in parts_bits], 0, T, tp)
    ref = exact.ring_rne(parts_bits, 0, T, tp)
    assert np.array_equal(got, ref)
    # a chunk that starts mid-shard gives the same rows
    r0 = T // tp + 2
    got2 = gemm.ring_sum([bf16.decode(p[r0:]) for p in parts_bits], r0, T, tp)
    assert np.array_equal(got2, ref[r0:])


def _rs(capacity, H, tp, T, a, w, cfg):
    m = manager.UserBufferModel(capacity, H, tp)
    assert m.set_active_shape((T, H)) == manager.OK
    k = a.shape[1]
    out = np.full((capacity, H), manager.CANARY, np.uint16)
    A = np.full((capacity, k), manager.CANARY, np.uint16)
    A[:T] = a
    st, written = gemm.rs_chunked(m, A, k, k, w, H, out, H, cfg)
    assert st == manager.OK and np.all(written == 1)
    assert np.all(out[T:] == manager.CANARY)
    return out[:T], m.ws[: tp * T * H].reshape(tp, T, H)


def test_ring_rs_schedule_free_and_shards():
    """The ring sum of a row depends only on its shard, never on chunking, streams, the
    method's chunk order or the rank; the partials are those of the ascending order."""
    rng = np.random.default_rng(31)
    T, H, K, tp = 48, 24, 256, 4
    a = wl.normal_bits(rng, (T, K))
    w = wl.normal_bits(rng, (K, H), 0.05)
    ref, ref_ws = _rs(64, H, tp, T, a, w, plan.OverlapCfg(method="bulk", num_splits=1,
                                                          reduce_order="ring"))
    asc, asc_ws = _rs(64, H, tp, T, a, w, plan.OverlapCfg(method="bulk", num_splits=1))
    assert np.array_equal(ref_ws, asc_ws)
    assert not np.array_equal(ref, asc)  # the per-hop rounding shows on random data
    for method in plan.METHODS:
        for ns in (2, 3, 5):
            for rank in (0, 3):
                cfg = plan.OverlapCfg(method=method, num_splits=ns, rank=rank, reduce_order="ring")
                got, _ = _rs(96, H, tp, T, a, w, cfg)
                assert np.array_equal(got, ref), (method, ns, rank)
    rows = np.array([0, 5, 11, 12, 30, 47])
    out_rows, _ = gemm.rs_rows_ring(rows, a[rows], w, T, tp)
    assert np.array_equal(out_rows, ref[rows])


def test_ring_equals_exact_when_every_hop_is_exact():
    """Small integer partials: every hop sum is an integer of magnitude <= 256, exact in
    bf16, so the ring order gives the exact sum."""
    rng = np.random.default_rng(32)
    T, H, K, tp = 32, 16, 64, 8  # slices of 8 terms in {-1, 0, 1}: partials in [-8, 8]
    a = wl.integer_bits(rng, (T, K), -1, 1)
    w = wl.integer_bits(rng, (K, H), -1, 1)
    ring, _ = _rs(32, H, tp, T, a, w, plan.OverlapCfg(method="pipeline", num_splits=2,
                                                      reduce_order="ring"))
    asc, _ = _rs(32, H, tp, T, a, w, plan.OverlapCfg(method="pipeline", num_splits=2))
    assert np.array_equal(ring, asc)


def test_tp1_ring_is_the_single_partial():
    rng = np.random.default_rng(33)
    a = wl.normal_bits(rng, (16, 64))
    w = wl.normal_bits(rng, (64, 8), 0.1)
    ring, ws = _rs(16, 8, 1, 16, a, w, plan.OverlapCfg(reduce_order="ring"))
    assert np.array_equal(ring, ws[0])


def test_unknown_reduce_order_is_rejected():
    m = manager.UserBufferModel(8, 8, 1)
    st, _ = gemm.rs_chunked(m, np.zeros((8, 8), np.uint16), 8, 8, np.zeros((8, 8), np.uint16), 8,
                            np.zeros((8, 8), np.uint16), 8, plan.OverlapCfg(reduce_order="tree"))
    assert st == manager.INVALID_ARG


def _ring_case(tp, shard):
    return [c for c in _golden() if c[0] == tp and c[1] == shard][0]


def test_planted_wrong_direction_is_caught(monkeypatch):
    """A ring walked the other way (from rank r-1 down to r) fails a hand-worked case."""
    def backwards(parts, row0, T, tp):
        bits = [bf16.encode_rne(p) for p in parts]
        r = row0 // (T // tp)
        acc = bits[(r - 1) % tp]
        for i in range(2, tp + 1):
            acc = gemm.ring_hop(acc, bits[(r - i) % tp])
        return acc

    monkeypatch.setattr(gemm, "ring_sum", backwards)
    with pytest.raises(AssertionError):
        test_hand_worked_cases(_ring_case(4, 0))


def test_planted_single_rounding_is_caught(monkeypatch):
    """Ring order without the rounding at each hop fails a hand-worked case."""
    def one_rounding(parts, row0, T, tp):
        r = row0 // (T // tp)
        acc = parts[(r + 1) % tp]
        for i in range(2, tp + 1):
            acc = acc + parts[(r + i) % tp]
        return bf16.encode_rne(acc)

    monkeypatch.setattr(gemm, "ring_sum", one_rounding)
    with pytest.raises(AssertionError):
        test_hand_worked_cases(_ring_case(4, 0))
