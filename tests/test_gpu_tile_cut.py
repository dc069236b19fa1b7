"""GPU parity of launches cut in two (the leading row bands that fill whole rounds of the
large tile, then the remaining rows with a smaller tile): bit-exact against the oracle on
integer inputs and bit for bit against the one-launch plan, on both sides.  The cuts are
forced through the handle's debug settings (ub_debug_set "cut_row"), so the tests do not
depend on the cost model; one test checks that the automatic plan does cut a launch whose
last round would be nearly empty, and ub_debug_last_plan shows every plan taken."""

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


def _force_cut(ub, h, cut, tile="256x256", tail="128x128"):
    gu.force_tile(ub, h, tile)
    ub.ub_debug_set(h, "cut_row", cut)
    m, n = map(int, tail.split("x"))
    ub.ub_debug_set(h, "tail_tile_m", m)
    ub.ub_debug_set(h, "tail_tile_n", n)


def _no_cut(ub, h, tile="256x256"):
    ub.ub_debug_set(h, "cut_row", 0)
    gu.force_tile(ub, h, tile)


@pytest.mark.parametrize("tile,tail", [("256x256", "128x128"), ("320x256", "128x256"),
                                       ("128x256", "256x256")])
@pytest.mark.parametrize("atomic", (False, True))
def test_cut_ag_integer_bit_exact(ub, atomic, tile, tail):
    """AG with the chip to itself (the device-side loop, or one host-loop stream), cut after
    the first 40 bands of the first tile (ragged rows after the cut).  Integer inputs: every
    element equals the oracle's, and equals the one-launch plan's."""
    rng = np.random.default_rng(61)
    cap, H, N, T = 13312, 264, 1280, 13216
    bm = int(tile.split("x")[0])
    cut = 40 * bm
    a = wl.integer_bits(rng, (T, H))
    wt = wl.integer_bits(rng, (H, N))
    reg = gu.Registration(ub, cap, H, 8, workspace=False, pad_rows=8)
    print(f"[cut ag] tile={tile} tail={tail} atomic={atomic} cut={cut}", flush=True)
    try:
        reg.set_T(T)
        reg.fill(a)
        method, ns = ("pipeline", 3) if atomic else ("bulk", 1)
        cfg = ub.make_cfg(method, ns, 1, atomic_gemm=atomic)
        m = om.UserBufferModel(cap, H, 8)
        assert m.set_active_shape((T, H)) == om.OK
        m.fill_active(a)
        ref = np.full((cap, N), om.CANARY, np.uint16)
        st, _ = og.ag_chunked(m, wt, N, N, ref, N, op.OverlapCfg(method=method, num_splits=ns,
                                                                 num_max_streams=1))
        assert st == om.OK
        w_t = gu.dev(wt)
        _force_cut(ub, reg.h, cut, tile, tail)
        c = gu.canary((cap + 8, N))
        ub.ub_gemm_ag_chunked(reg.h, w_t, N, N, c, N, cfg)
        torch.cuda.synchronize()
        tm, tn = map(int, tile.split("x"))
        sm, sn = map(int, tail.split("x"))
        assert ub.ub_debug_last_plan(reg.h) == (tm, tn, cut, sm, sn)
        got = gu.host(c)
        assert np.array_equal(got[:T], ref[:T])
        assert np.all(got[T:] == gu.CANARY)
        _no_cut(ub, reg.h, tile)
        c.fill_(gu.CANARY)
        ub.ub_gemm_ag_chunked(reg.h, w_t, N, N, c, N, cfg)
        torch.cuda.synchronize()
        assert ub.ub_debug_last_plan(reg.h)[2] == -1
        assert np.array_equal(gu.host(c), got)
    finally:
        reg.close()


def test_no_cut_with_several_streams(ub):
    """Launches that share the chip with other streams are never cut by the cost model."""
    rng = np.random.default_rng(63)
    cap, H, N = 30720, 256, 1280
    reg = gu.Registration(ub, cap, H, 8, workspace=False, pad_rows=8)
    try:
        reg.fill(wl.integer_bits(rng, (cap, H)))
        w_t = gu.dev(wl.integer_bits(rng, (H, N)))
        c = gu.canary((cap + 8, N))
        for T in (13216, 17280, 26424, 30720):
            reg.set_T(T)
            ub.ub_gemm_ag_chunked(reg.h, w_t, N, N, c, N, ub.make_cfg("pipeline", 3, 3))
            torch.cuda.synchronize()
            assert ub.ub_debug_last_plan(reg.h)[2] < 0, T
    finally:
        reg.close()


def test_automatic_plan_cuts_a_nearly_empty_last_round(ub):
    """With the chip to itself, some launch of the GQA column count (1280) over a T sweep
    is cut by the cost model (a last round holding only a few tiles), and the cut output
    equals the one-launch plan's bit for bit."""
    rng = np.random.default_rng(64)
    cap, H, N = 30720, 256, 1280
    reg = gu.Registration(ub, cap, H, 8, workspace=False, pad_rows=8)
    try:
        reg.fill(wl.normal_bits(rng, (cap, H)))
        w_t = gu.dev(wl.normal_bits(rng, (H, N), 0.02))
        c = gu.canary((cap + 8, N))
        cut_T = None
        for T in range(13056, 30721, 1016):
            reg.set_T(T)
            ub.ub_gemm_ag_chunked(reg.h, w_t, N, N, c, N, ub.make_cfg("bulk", 8, atomic_gemm=True))
            torch.cuda.synchronize()
            plan = ub.ub_debug_last_plan(reg.h)
            if plan[2] >= 0:
                cut_T = T
                print(f"[auto cut] T={T} plan={plan}", flush=True)
                break
        assert cut_T is not None, "no automatic cut over the sweep"
        got = gu.host(c)
        tm, tn = ub.ub_debug_last_plan(reg.h)[:2]
        gu.force_tile(ub, reg.h, f"{tm}x{tn}")
        c.fill_(gu.CANARY)
        ub.ub_gemm_ag_chunked(reg.h, w_t, N, N, c, N, ub.make_cfg("bulk", 8, atomic_gemm=True))
        torch.cuda.synchronize()
        assert np.array_equal(gu.host(c), got)
    finally:
        reg.close()


@pytest.mark.parametrize("fuse", (False, True))
@pytest.mark.parametrize("order", ("ascending", "ring"))
@pytest.mark.parametrize("atomic", (False, True))
def test_cut_rs_integer_bit_exact(ub, fuse, order, atomic):
    """RS, 8 slices, one launch with the chip to itself, cut after 32 bands of 256 rows: the
    separate and the fused sums both equal the oracle's on integer inputs, in either
    order, as do the partials; the fused counters are left at zero."""
    rng = np.random.default_rng(62)
    cap, H, tp, T = 8448, 256, 8, 8448
    K = tp * 64
    a = wl.integer_bits(rng, (T, K))
    wt = wl.integer_bits(rng, (K, H))
    reg = gu.Registration(ub, cap, H, tp, pad_rows=8)
    print(f"[cut rs] fuse={fuse} order={order} atomic={atomic}", flush=True)
    try:
        reg.set_T(T)
        m = om.UserBufferModel(cap, H, tp)
        assert m.set_active_shape((T, H)) == om.OK
        ref = np.full((cap, H), om.CANARY, np.uint16)
        method, ns = ("pipeline", 3) if atomic else ("bulk", 1)
        st, _ = og.rs_chunked(m, a, K, K, wt, H, ref, H,
                              op.OverlapCfg(method=method, num_splits=ns, num_max_streams=1,
                                            reduce_order=order))
        assert st == om.OK
        _force_cut(ub, reg.h, 32 * 256)
        out = gu.canary((cap + 8, H))
        cfg = ub.make_cfg(method, ns, 1, atomic_gemm=atomic, reduce_order=order, fuse_reduce=fuse)
        ub.ub_gemm_rs_chunked(reg.h, gu.dev(a), K, K, gu.dev(wt), H, out, H, cfg)
        torch.cuda.synchronize()
        assert ub.ub_debug_last_plan(reg.h) == (256, 256, 32 * 256, 128, 128)
        got = gu.host(out)
        assert np.array_equal(got[:T], ref[:T])
        assert np.all(got[T:] == gu.CANARY)
        ws = gu.host(reg.ws_t)
        assert np.array_equal(ws[: tp * T * H].reshape(tp, T, H), m.ws[: tp * T * H].reshape(tp, T, H))
        assert reg.counters_clean()
    finally:
        reg.close()


def test_cut_gqa_single_launch_matches(ub):
    """The GQA-bulk shape (hidden 8192, 1280 columns) at T = 13216 in the device-side loop
    with the automatic plan, and the same with a forced cut after 51 bands of 256 rows:
    both equal the one-launch 256 x 256 plan bit for bit, and rows around the cut match the
    oracle within the gate."""
    w = wl.gqa_bulk()
    ra, rw, _ = w.seeds()
    T = 13216
    a = wl.activations(w, T, ra)
    wt = wl.weights(w, rw)
    reg = gu.Registration(ub, w.capacity, w.hidden, w.tp, workspace=False, pad_rows=8)
    try:
        reg.set_T(T)
        reg.fill(a)
        cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, atomic_gemm=True)
        w_t = gu.dev(wt)
        N = w.n_cols
        c = gu.canary((w.capacity + 8, N))
        ub.ub_gemm_ag_chunked(reg.h, w_t, N, N, c, N, cfg)
        torch.cuda.synchronize()
        print(f"[gqa cut] automatic plan {ub.ub_debug_last_plan(reg.h)}", flush=True)
        auto = gu.host(c)
        assert np.all(auto[T:] == gu.CANARY)
        _force_cut(ub, reg.h, 51 * 256)
        c.fill_(gu.CANARY)
        ub.ub_gemm_ag_chunked(reg.h, w_t, N, N, c, N, cfg)
        torch.cuda.synchronize()
        got = gu.host(c)
        assert np.array_equal(got, auto)
        _no_cut(ub, reg.h)
        c.fill_(gu.CANARY)
        ub.ub_gemm_ag_chunked(reg.h, w_t, N, N, c, N, cfg)
        torch.cuda.synchronize()
        assert np.array_equal(gu.host(c), got)
        rows = np.array([0, 51 * 256 - 1, 51 * 256, 51 * 256 + 127, 51 * 256 + 128, T - 1])
        gu.check_close(got[rows], og.ag_rows(a[rows], wt), a[rows], wt, "gqa cut rows")
    finally:
        reg.close()
