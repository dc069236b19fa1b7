"""GPU test of ub_gemm_rs_chunked_noalloc, the reduce-scatter entry point that allocates
nothing (its partial slots and fused-sum counters live in the library's fixed device
scratch): called through the C ABI, its output equals ub_gemm_rs_chunked's on a handle with
a registered workspace, bit for bit, and the oracle's on integer inputs, on two calls in a
row, the second with a smaller T; for the separate and the fused sum, both summation
orders, the host loop and the device-side loop.  Requests beyond the scratch's 32 MiB are
rejected before anything is enqueued."""

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


def _oracle(cap, H, tp, a_bits, w_bits, cfg):
    T, k = a_bits.shape
    m = om.UserBufferModel(cap, H, tp)
    assert m.set_active_shape((T, H)) == om.OK
    out = np.full((cap, H), om.CANARY, np.uint16)
    st, _ = og.rs_chunked(m, a_bits, k, k, w_bits, H, out, H, cfg)
    assert st == om.OK
    return out[:T]


@pytest.mark.parametrize("fuse", (False, True))
def test_noalloc_matches_workspace_entry_point(ub, fuse):
    rng = np.random.default_rng(160)
    cap, H, tp = 1024, 264, 8
    K = tp * 136
    a = wl.integer_bits(rng, (cap, K))
    w = wl.integer_bits(rng, (K, H))
    a_r = wl.normal_bits(rng, (cap, K))
    w_r = wl.normal_bits(rng, (K, H), 0.02)
    reg = gu.Registration(ub, cap, H, tp, pad_rows=8)
    bare = gu.Registration(ub, cap, H, tp, workspace=False)  # no workspace at all
    try:
        for T in (1024, 600):  # two calls in a row, the second smaller
            reg.set_T(T)
            bare.set_T(T)
            for order in ("ascending", "ring"):
                want = _oracle(cap, H, tp, a[:T], w, op.OverlapCfg(method="pipeline", num_splits=3,
                                                                   reduce_order=order))
                for atomic in (False, True):
                    print(f"[noalloc] fuse={fuse} T={T} {order} atomic={atomic}", flush=True)
                    cfg = ub.make_cfg("pipeline", 3, atomic_gemm=atomic, reduce_order=order, fuse_reduce=fuse)
                    for bits_a, bits_w, exact in ((a, w, True), (a_r, w_r, False)):
                        at, wt = gu.dev(bits_a[:T]), gu.dev(bits_w)
                        ref = gu.canary((cap + 8, H))
                        ub.ub_gemm_rs_chunked(reg.h, at, K, K, wt, H, ref, H, cfg)
                        for h in (reg.h, bare.h):
                            got = gu.canary((cap + 8, H))
                            ub.ub_gemm_rs_chunked_noalloc(h, at, K, K, wt, H, got, H, cfg)
                            torch.cuda.synchronize()
                            assert torch.equal(got, ref), (T, order, atomic)
                            g = gu.host(got)
                            assert np.all(g[T:] == gu.CANARY)
                            if exact:
                                assert np.array_equal(g[:T], want), (T, order, atomic)
        assert reg.counters_clean()
    finally:
        reg.close()
        bare.close()


def test_noalloc_rejects_beyond_scratch(ub):
    """tp * T * hidden * 2 bytes of partials over 32 MiB: UB_ERR_BUFFER_TOO_SMALL, nothing
    enqueued (the output stays canary); just under it runs."""
    H, tp = 4096, 8
    cap = 1024
    reg = gu.Registration(ub, cap, H, tp, workspace=False)
    try:
        a = torch.zeros((cap, tp * 64), dtype=torch.int16, device="cuda")
        w = torch.zeros((tp * 64, H), dtype=torch.int16, device="cuda")
        out = gu.canary((cap, H))
        cfg = ub.make_cfg("pipeline", 2, atomic_gemm=True)
        reg.set_T(cap)  # 8 * 1024 * 4096 * 2 = 64 MiB of partials
        with pytest.raises(ub.UBError) as e:
            ub.ub_gemm_rs_chunked_noalloc(reg.h, a, tp * 64, tp * 64, w, H, out, H, cfg)
        assert e.value.name == "UB_ERR_BUFFER_TOO_SMALL"
        torch.cuda.synchronize()
        assert bool((out == gu.CANARY).all().item())
        reg.set_T(512)  # 32 MiB exactly, no counters: fits
        ub.ub_gemm_rs_chunked_noalloc(reg.h, a, tp * 64, tp * 64, w, H, out, H, cfg)
        torch.cuda.synchronize()
        assert bool((out[:512] == 0).all().item()) and bool((out[512:] == gu.CANARY).all().item())
        cfg = ub.make_cfg("pipeline", 2, atomic_gemm=True, fuse_reduce=True)  # + counters: too big
        with pytest.raises(ub.UBError) as e:
            ub.ub_gemm_rs_chunked_noalloc(reg.h, a, tp * 64, tp * 64, w, H, out, H, cfg)
        assert e.value.name == "UB_ERR_BUFFER_TOO_SMALL"
    finally:
        reg.close()
