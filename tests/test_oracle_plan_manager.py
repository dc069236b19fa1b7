"""Pins of the oracle's buffer-manager model and chunk plan against the pages' statements
(golden fixtures under tests/golden/, each citing its page and section)."""

import itertools
import os

import pytest

from oracle import manager, plan

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield [part.split() for part in line.split("|")]


def constraint_cases():
    out = []
    for reg, shape, exp in _rows("active_shape_constraints.txt"):
        cap, hid, tp = map(int, reg)
        out.append((cap, hid, tp, tuple(int(x) for x in shape[0].split(",")), exp[0]))
    return out


def option_cases():
    out = []
    for lhs, rhs in _rows("overlap_options.txt"):
        method, ns, nms, agg, tp, op = lhs
        out.append((method, int(ns), None if nms == "default" else int(nms), bool(int(agg)),
                    int(tp), op, tuple(int(x) for x in rhs)))
    return out


@pytest.mark.parametrize("cap,hid,tp,shape,expected", constraint_cases())
def test_active_shape_constraints(cap, hid, tp, shape, expected):
    m = manager.UserBufferModel(cap, hid, tp)
    m.set_active_shape((cap // 2 // tp * tp or tp, hid))
    before = m.active_shape
    st = m.set_active_shape(shape)
    assert st == expected
    if st != manager.OK:
        assert m.active_shape == before  # a rejected request changes nothing
    else:
        assert m.active_shape == (shape[0], hid)
    assert m.capacity_shape == (cap, hid)
    assert m.ub.size == cap * hid  # never reallocated


def test_registration_rules():
    assert manager.check_registration(512, 256, 2) == manager.OK
    assert manager.check_registration(512, 256, 2, "fp8") == manager.DTYPE
    assert manager.check_registration(512, 256, 2, "fp8_e5m2") == manager.DTYPE
    assert manager.check_registration(512, 256, 2, "fp8_e4m3") == manager.OK
    assert manager.check_registration(0, 256, 2) == manager.INVALID_ARG
    assert manager.check_registration(512, 0, 2) == manager.INVALID_ARG
    assert manager.check_registration(512, 256, 0) == manager.INVALID_ARG
    assert manager.check_registration(510, 256, 4) == manager.TP_DIVISIBILITY
    m = manager.UserBufferModel(512, 256, 2)
    assert m.active_shape == m.capacity_shape == (512, 256)  # starts at capacity


def test_buffer_sized_by_communicated_tensor():
    """[MLM#1240]: the buffer holds the communicated [S, H] activations, not the
    expanded GEMM output: its size does not depend on the output width."""
    m = manager.UserBufferModel(8192, 4096, 8)
    assert m.ub.size == 8192 * 4096
    assert m.ws.size == 8 * 8192 * 4096


def test_offsets_follow_active_T():
    m = manager.UserBufferModel(16384, 4096, 8)
    assert m.set_active_shape((12280, 4096)) == manager.OK
    assert m.shard_rows == 1535
    assert m.shard_offset_elems(3) == 3 * 1535 * 4096
    assert m.partial_offset_elems(2, 100) == (2 * 12280 + 100) * 4096
    assert m.row_offset_elems(3070) == 3070 * 4096
    assert m.copy_in([0] * (1535 * 4096), 1535, 7 * 1535) == manager.OK
    assert m.copy_in([0] * 4096, 1, 12280) == manager.INVALID_ARG  # past active T


@pytest.mark.parametrize("method,ns,nms,agg,tp,op,expected", option_cases())
def test_option_semantics(method, ns, nms, agg, tp, op, expected):
    kw = dict(method=method, num_splits=ns, aggregate=agg)
    if nms is not None:
        kw["num_max_streams"] = nms
    cfg = plan.OverlapCfg(**kw)
    eff, units, streams = expected
    assert plan.effective_splits(cfg, tp) == eff
    p = plan.build(8 * tp * 16, tp, cfg, op)
    assert len(p) == units
    assert len({u.stream for u in p}) == streams == plan.num_streams(cfg, tp)


def _check_plan(T, tp, cfg, op):
    p = plan.build(T, tp, cfg, op)
    n = plan.effective_splits(cfg, tp)
    S = plan.num_streams(cfg, tp)
    covered = []
    for j, u in enumerate(p):
        assert u.pos == j and u.stream == j % S
        covered.extend(range(u.row0, u.row1))
    assert sorted(covered) == list(range(T))            # every row exactly once
    assert sorted(u.index for u in p) == list(range(len(p)))
    bounds = plan.chunk_rows(T, n)
    assert bounds[0][0] == 0 and bounds[-1][1] == T
    assert all(b - a in (T // n, T // n + 1) for a, b in bounds)
    return p


def test_plan_exhaustive_small():
    for T, tp in itertools.product((8, 16, 24, 40, 56, 96), (1, 2, 4, 8)):
        if T % tp:
            continue
        for method, ns, nms, agg, rank, op in itertools.product(
                plan.METHODS, (1, 2, 3, 4, 5, 8), (1, 2, 3, 8), (False, True), (0, 1, tp - 1), ("ag", "rs")):
            cfg = plan.OverlapCfg(method=method, num_splits=ns, num_max_streams=nms,
                                  aggregate=agg, rank=rank)
            p = _check_plan(T, tp, cfg, op)
            U = len(p)
            if method == plan.RING and op == "ag":
                home = rank // (2 if agg else 1)
                assert [u.index for u in p] == [(home - i) % U for i in range(U)]
            elif method == plan.RING:
                assert p[-1].index == rank % U  # own shard finished last
            else:
                assert [u.index for u in p] == list(range(U))


def test_tiny_and_real_plans():
    # tiny: ring over tp = 2 -> 2 chunks of 128 rows, 2 streams
    p = plan.build(256, 2, plan.OverlapCfg(num_splits=2), "ag")
    assert [(u.row0, u.row1, u.stream) for u in p] == [(0, 128, 0), (128, 256, 1)]
    # fc1: ring over 8 with aggregate -> 4 units of 2T/8 rows, 3 streams
    p = plan.build(16384, 8, plan.OverlapCfg(num_splits=8, aggregate=True), "ag")
    assert [(u.row1 - u.row0) for u in p] == [4096] * 4 and [u.stream for u in p] == [0, 1, 2, 0]
    # fc2: pipeline, 4 chunks of T/4 at T = 12280 -> 3070 rows each
    p = plan.build(12280, 8, plan.OverlapCfg(method="pipeline", num_splits=4), "rs")
    assert [(u.row0, u.row1) for u in p] == [(0, 3070), (3070, 6140), (6140, 9210), (9210, 12280)]
