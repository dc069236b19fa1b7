"""GPU parity of the fused reduce-scatter sum (fuse_reduce=1: the last slice tile of each
output tile sums the tp partials inside the slice-GEMM launch) against the oracle and
against the separate reduction launch, which must give the same bits."""

import numpy as np
import pytest
import torch

from chunked_tp_overlap_amd import workloads as wl
from oracle import gemm as og
from oracle import manager as om
from oracle import plan as op
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ub():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import chunked_tp_overlap_amd.ub as m
    return m


def _run(ub, reg, a_t, k, w_t, cfg, ldo=None, extra_rows=8):
    H = reg.hidden
    ldo = ldo or H
    out = gu.canary((reg.capacity + extra_rows, ldo))
    ub.ub_gemm_rs_chunked(reg.h, a_t, k, k, w_t, H, out, ldo, cfg)
    torch.cuda.synchronize()
    return gu.host(out)


def _oracle_rs(capacity, H, tp, a_bits, w_bits, cfg):
    T, k = a_bits.shape
    m = om.UserBufferModel(capacity, H, tp)
    assert m.set_active_shape((T, H)) == om.OK
    out = np.full((capacity, H), om.CANARY, np.uint16)
    st, written = og.rs_chunked(m, a_bits, k, k, w_bits, H, out, H, cfg)
    assert st == om.OK and np.all(written == 1)
    return out[:T], m.ws[: tp * T * H].reshape(tp, T, H)


@pytest.mark.parametrize("cap,H,K,T,tp,method,ns", [
    (512, 256, 256, 256, 2, "ring_exchange", 2),
    (1024, 512, 1024, 296, 8, "pipeline", 4),       # 8 slices of 128, ragged chunks
    (256, 64, 1024, 96, 4, "bulk", 5),
    (64, 128, 512, 64, 1, "pipeline", 2),            # tp = 1: each tile is its own last slice
    (768, 136, 768, 294, 6, "ring_exchange", 6),     # tp = 6: the run-time slot count
])
def test_fused_integer_inputs_bit_exact(ub, cap, H, K, T, tp, method, ns):
    """Integer inputs (exact partials): the fused sum equals the oracle's reduce-scatter
    bit for bit in both orders, host loop and device-side loop, and the partials left in
    the workspace are the oracle's."""
    rng = np.random.default_rng(cap + H + K + T + 1)
    a = wl.integer_bits(rng, (T, K))
    wt = wl.integer_bits(rng, (K, H))
    print(f"[fused int] cap={cap} H={H} K={K} T={T} tp={tp} {method} ns={ns}", flush=True)
    reg = gu.Registration(ub, cap, H, tp, pad_rows=8)
    try:
        reg.set_T(T)
        for order in ("ascending", "ring"):
            ref, parts = _oracle_rs(cap, H, tp, a, wt, op.OverlapCfg(method=method, num_splits=ns,
                                                                     reduce_order=order))
            for atomic in (False, True):
                reg.ws_t.fill_(gu.CANARY)
                cfg = ub.make_cfg(method, ns, atomic_gemm=atomic, reduce_order=order, fuse_reduce=True)
                out = _run(ub, reg, gu.dev(a), K, gu.dev(wt), cfg)
                assert np.array_equal(out[:T], ref), (order, atomic)
                ws = gu.host(reg.ws_t)
                assert np.array_equal(ws[: tp * T * H].reshape(tp, T, H), parts)
                assert np.all(ws[tp * T * H:] == gu.CANARY)
                assert np.all(out[T:] == gu.CANARY)
    finally:
        reg.close()


@pytest.mark.parametrize("tile", gu.BF16_TILES)
def test_fused_every_tile_shape(ub, tile):
    """Each GEMM tile shape, forced: the fused sum is bit-exact against the oracle on
    integer inputs (ragged rows, ragged last column tile, tp = 8) in both orders."""
    rng = np.random.default_rng(24)
    cap, H, K, T, tp = 1024, 264, 2048, 600, 8
    a = wl.integer_bits(rng, (T, K))
    wt = wl.integer_bits(rng, (K, H))
    print(f"[fused tile {tile}] cap={cap} H={H} K={K} T={T}", flush=True)
    reg = gu.Registration(ub, cap, H, tp, pad_rows=8)
    gu.force_tile(ub, reg.h, tile)
    try:
        reg.set_T(T)
        for order in ("ascending", "ring"):
            ref, _ = _oracle_rs(cap, H, tp, a, wt, op.OverlapCfg(method="pipeline", num_splits=3,
                                                                 reduce_order=order))
            for atomic in (False, True):
                cfg = ub.make_cfg("pipeline", 3, atomic_gemm=atomic, reduce_order=order,
                                  fuse_reduce=True)
                out = _run(ub, reg, gu.dev(a), K, gu.dev(wt), cfg)
                assert np.array_equal(out[:T], ref), (order, atomic)
                assert np.all(out[T:] == gu.CANARY)
    finally:
        reg.close()


def test_fused_equals_separate_reduction_every_schedule(ub):
    """Random inputs: for every schedule and both orders, the fused call gives the bits of
    the separate reduction, and the counters are left ready for the next call (calls at
    changing T on one registration, each checked)."""
    rng = np.random.default_rng(25)
    H, K, tp = 136, 1024, 8
    cap = 512
    a = gu.dev(wl.normal_bits(rng, (cap, K)))
    wt = gu.dev(wl.normal_bits(rng, (K, H), 0.02))
    reg = gu.Registration(ub, cap, H, tp)
    try:
        for T in (240, 96, 512, 240):
            reg.set_T(T)
            print(f"[fused schedules] T={T}", flush=True)
            for order in ("ascending", "ring"):
                ref = _run(ub, reg, a, K, wt, ub.make_cfg("pipeline", 1, reduce_order=order))[:T]
                for method in ("ring_exchange", "pipeline", "bulk"):
                    for ns in (1, 3, 4):
                        for atomic in (False, True):
                            cfg = ub.make_cfg(method, ns, 3, atomic_gemm=atomic, rank=5,
                                              reduce_order=order, fuse_reduce=True)
                            got = _run(ub, reg, a, K, wt, cfg)
                            assert np.array_equal(got[:T], ref), (T, order, method, ns, atomic)
                            assert np.all(got[T:] == gu.CANARY)
            assert reg.counters_clean(), T
    finally:
        reg.close()


def test_fused_strided_output_rows(ub):
    """ldo > H: the fused sum writes only the first H columns of each output row."""
    rng = np.random.default_rng(26)
    T, H, K, tp, ldo = 200, 200, 1024, 8, 232
    a = gu.dev(wl.normal_bits(rng, (T, K)))
    wt = gu.dev(wl.normal_bits(rng, (K, H), 0.02))
    reg = gu.Registration(ub, 256, H, tp)
    try:
        reg.set_T(T)
        ref = _run(ub, reg, a, K, wt, ub.make_cfg("pipeline", 3))[:T]
        for atomic in (False, True):
            oh = _run(ub, reg, a, K, wt, ub.make_cfg("pipeline", 3, atomic_gemm=atomic, fuse_reduce=True),
                      ldo=ldo, extra_rows=3)
            assert np.array_equal(oh[:T, :H], ref), atomic
            assert np.all(oh[:T, H:] == gu.CANARY) and np.all(oh[T:] == gu.CANARY)
    finally:
        reg.close()


def test_fused_fc2_full_size(ub):
    """The MLP fc2 workload (capacity 16384, hidden 4096, K 14336 in 8 slices) over its T
    sweep on one registration, pipeline on 3 streams and the device-side loop: the fused
    output equals the separate reduction's bit for bit, and sampled rows (chunk and shard
    boundaries) match the oracle within the gate."""
    w = wl.fc2()
    ra, rw, _ = w.seeds()
    a_all = wl.activations(w, w.capacity, ra)
    wt = wl.weights(w, rw)
    a_t, w_t = gu.dev(a_all), gu.dev(wt)
    H, tp = w.hidden, w.tp
    reg = gu.Registration(ub, w.capacity, H, tp, pad_rows=8)
    rng = np.random.default_rng(27)
    try:
        ref = gu.canary((w.capacity + 8, H))
        got = gu.canary((w.capacity + 8, H))
        for T in wl.FC2_TOKENS:
            reg.set_T(T)
            for atomic in (False, True):
                print(f"[fused fc2] T={T} atomic={atomic}", flush=True)
                base = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, atomic_gemm=atomic)
                fused = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, atomic_gemm=atomic,
                                    fuse_reduce=True)
                ref.fill_(gu.CANARY)
                got.fill_(gu.CANARY)
                ub.ub_gemm_rs_chunked(reg.h, a_t, w.k, w.k, w_t, H, ref, H, base)
                ub.ub_gemm_rs_chunked(reg.h, a_t, w.k, w.k, w_t, H, got, H, fused)
                torch.cuda.synchronize()
                assert torch.equal(got, ref), (T, atomic)
            oh = gu.host(got)
            rows = set(rng.integers(0, T, size=12).tolist()) | {0, T - 1}
            for c in range(1, w.num_splits):
                rows |= {(c * T) // w.num_splits - 1, (c * T) // w.num_splits}
            for r in range(1, tp):
                rows |= {r * T // tp - 1, r * T // tp}
            rows = np.array(sorted(rows))
            want, _ = og.rs_rows(a_all[rows], wt, tp)
            gu.check_rs_close(oh[rows], want, a_all[rows], wt, tp, f"fused fc2 T={T}")
            assert np.all(oh[T:] == gu.CANARY)
        assert reg.counters_clean()
    finally:
        reg.close()
