"""GPU parity of launches cut in two (the leading row bands that fill whole rounds of the
large tile, then the remaining rows with a smaller tile): bit-exact against the oracle on
integer inputs and bit for bit against the one-launch plan, on both sides.  The tile plan
log (UBX_GEMM_LOG) shows that the cut was taken."""

import os

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


def _plans(path):
    with open(path) as f:
        rows = [dict(kv.split("=") for kv in line.split()) for line in f if line.strip()]
    os.remove(path)
    return rows


@pytest.mark.parametrize("atomic", (False, True))
def test_cut_ag_integer_bit_exact(ub, tmp_path, monkeypatch, atomic):
    """AG with the chip to itself (the device-side loop, or one host-loop stream): 13216
    rows x 1280 columns make 260 tiles of 256 x 256, so the plan runs 51 bands in one round
    and the last 160 rows as 128 x 128 tiles.  Integer inputs: every element equals the
    oracle's, and equals the one-launch plan's."""
    rng = np.random.default_rng(61)
    cap, H, N, T = 13312, 256, 1280, 13216
    a = wl.integer_bits(rng, (T, H))
    wt = wl.integer_bits(rng, (H, N))
    log = str(tmp_path / "plans.txt")
    reg = gu.Registration(ub, cap, H, 8, workspace=False, pad_rows=8)
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
        monkeypatch.setenv("UBX_GEMM_LOG", log)
        c = gu.canary((cap + 8, N))
        ub.ub_gemm_ag_chunked(reg.h, w_t, N, N, c, N, cfg)
        torch.cuda.synchronize()
        plans = _plans(log)
        assert len(plans) == 1 and int(plans[0]["cut"]) == 51 * 256, plans
        got = gu.host(c)
        assert np.array_equal(got[:T], ref[:T])
        assert np.all(got[T:] == gu.CANARY)
        monkeypatch.delenv("UBX_GEMM_LOG")
        monkeypatch.setenv("UBX_GEMM_TILE", "256x256")
        c.fill_(gu.CANARY)
        ub.ub_gemm_ag_chunked(reg.h, w_t, N, N, c, N, cfg)
        torch.cuda.synchronize()
        assert np.array_equal(gu.host(c), got)
    finally:
        reg.close()


def test_no_cut_with_several_streams(ub, tmp_path, monkeypatch):
    """Launches that share the chip with other streams are never cut."""
    rng = np.random.default_rng(63)
    cap, H, N, T = 13824, 256, 1280, 13824
    log = str(tmp_path / "plans.txt")
    reg = gu.Registration(ub, cap, H, 8, workspace=False, pad_rows=8)
    try:
        reg.set_T(T)
        reg.fill(wl.integer_bits(rng, (T, H)))
        monkeypatch.setenv("UBX_GEMM_LOG", log)
        c = gu.canary((cap + 8, N))
        ub.ub_gemm_ag_chunked(reg.h, gu.dev(wl.integer_bits(rng, (H, N))), N, N, c, N,
                              ub.make_cfg("pipeline", 3, 3))
        torch.cuda.synchronize()
        plans = _plans(log)
        assert len(plans) == 3 and all(int(p["cut"]) < 0 for p in plans), plans
    finally:
        reg.close()


@pytest.mark.parametrize("fuse", (False, True))
@pytest.mark.parametrize("order", ("ascending", "ring"))
@pytest.mark.parametrize("atomic", (False, True))
def test_cut_rs_integer_bit_exact(ub, tmp_path, monkeypatch, fuse, order, atomic):
    """RS, 8 slices, one launch with the chip to itself: 8448 rows x 256 columns x 8 slices
    make 264 tiles, cut after 32 bands; the separate and the fused sums both equal the
    oracle's on integer inputs, in either order, as do the partials."""
    rng = np.random.default_rng(62)
    cap, H, tp, T = 8448, 256, 8, 8448
    K = tp * 64
    a = wl.integer_bits(rng, (T, K))
    wt = wl.integer_bits(rng, (K, H))
    log = str(tmp_path / "plans.txt")
    reg = gu.Registration(ub, cap, H, tp, pad_rows=8)
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
        monkeypatch.setenv("UBX_GEMM_LOG", log)
        out = gu.canary((cap + 8, H))
        cfg = ub.make_cfg(method, ns, 1, atomic_gemm=atomic, reduce_order=order, fuse_reduce=fuse)
        ub.ub_gemm_rs_chunked(reg.h, gu.dev(a), K, K, gu.dev(wt), H, out, H, cfg)
        torch.cuda.synchronize()
        plans = _plans(log)
        assert len(plans) == 1 and int(plans[0]["cut"]) == 32 * 256, plans
        got = gu.host(out)
        assert np.array_equal(got[:T], ref[:T])
        assert np.all(got[T:] == gu.CANARY)
        ws = gu.host(reg.ws_t)
        assert np.array_equal(ws[: tp * T * H].reshape(tp, T, H), m.ws[: tp * T * H].reshape(tp, T, H))
    finally:
        reg.close()


def test_cut_gqa_single_launch_matches(ub, tmp_path, monkeypatch):
    """The GQA-bulk shape (hidden 8192, 1280 columns) at T = 13216 in the device-side loop:
    260 tiles of 256 x 256 on 256 CUs, so the plan cuts after 51 bands.  The output equals
    the one-launch plan's bit for bit, and rows around the cut match the oracle within
    the gate."""
    w = wl.gqa_bulk()
    ra, rw, _ = w.seeds()
    T = 13216
    a = wl.activations(w, T, ra)
    wt = wl.weights(w, rw)
    log = str(tmp_path / "plans.txt")
    reg = gu.Registration(ub, w.capacity, w.hidden, w.tp, workspace=False, pad_rows=8)
    try:
        reg.set_T(T)
        reg.fill(a)
        cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, atomic_gemm=True)
        w_t = gu.dev(wt)
        N = w.n_cols
        monkeypatch.setenv("UBX_GEMM_LOG", log)
        c = gu.canary((w.capacity + 8, N))
        ub.ub_gemm_ag_chunked(reg.h, w_t, N, N, c, N, cfg)
        torch.cuda.synchronize()
        plans = _plans(log)
        assert len(plans) == 1 and int(plans[0]["cut"]) == 51 * 256, plans
        got = gu.host(c)
        assert np.all(got[T:] == gu.CANARY)
        monkeypatch.delenv("UBX_GEMM_LOG")
        monkeypatch.setenv("UBX_GEMM_TILE", "256x256")
        c.fill_(gu.CANARY)
        ub.ub_gemm_ag_chunked(reg.h, w_t, N, N, c, N, cfg)
        torch.cuda.synchronize()
        assert np.array_equal(gu.host(c), got)
        rows = np.array([0, 51 * 256 - 1, 51 * 256, 51 * 256 + 127, 51 * 256 + 128, T - 1])
        gu.check_close(got[rows], og.ag_rows(a[rows], wt), a[rows], wt, "gqa cut rows")
    finally:
        reg.close()
