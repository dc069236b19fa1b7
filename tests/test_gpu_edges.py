"""GPU edge cases of the chunked GEMMs against the oracle: empty chunks (more chunks than
rows), a single active row, the largest tp (64 ring chunks through the device-side loop's
64-unit table), one row per shard in both reduction orders, and T == capacity at the
largest registration of the workloads."""

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


def _ag(ub, reg, a, w, cfg_kw):
    T, H = a.shape
    N = w.shape[1]
    reg.set_T(T)
    reg.fill(a)
    c = gu.canary((reg.capacity + 4, N))
    ub.ub_gemm_ag_chunked(reg.h, gu.dev(w), N, N, c, N, ub.make_cfg(**cfg_kw))
    torch.cuda.synchronize()
    return gu.host(c)


def _ag_oracle(cap, tp, a, w, cfg):
    T, H = a.shape
    m = om.UserBufferModel(cap, H, tp)
    assert m.set_active_shape((T, H)) == om.OK
    m.fill_active(a)
    N = w.shape[1]
    c = np.full((cap, N), om.CANARY, np.uint16)
    st, written = og.ag_chunked(m, w, N, N, c, N, cfg)
    assert st == om.OK and np.all(written == 1)
    return c[:T]


@pytest.mark.parametrize("cap,H,N,T,tp,method,ns", [
    (64, 128, 72, 8, 8, "pipeline", 13),     # 13 chunks over 8 rows: 5 chunks are empty
    (64, 64, 8, 1, 1, "bulk", 4),            # one active row, three empty chunks
    (4096, 128, 136, 512, 64, "ring_exchange", 1),  # tp = 64: 64 ring chunks of 8 rows
])
def test_ag_edges_bit_exact(ub, cap, H, N, T, tp, method, ns):
    rng = np.random.default_rng(cap + T + tp)
    a = wl.integer_bits(rng, (T, H))
    w = wl.integer_bits(rng, (H, N))
    print(f"[edge ag] cap={cap} H={H} N={N} T={T} tp={tp} {method} ns={ns}", flush=True)
    reg = gu.Registration(ub, cap, H, tp, workspace=False, pad_rows=4)
    try:
        want = _ag_oracle(cap, tp, a, w, op.OverlapCfg(method=method, num_splits=ns))
        for atomic in (False, True):
            for rank in (0, tp - 1):
                got = _ag(ub, reg, a, w, dict(method=method, num_splits=ns, atomic_gemm=atomic, rank=rank))
                assert np.array_equal(got[:T], want), (atomic, rank)
                assert np.all(got[T:] == gu.CANARY)
    finally:
        reg.close()


@pytest.mark.parametrize("tp,T,order", [(8, 8, "ascending"), (8, 8, "ring"), (64, 64, "ascending"),
                                        (64, 64, "ring"), (4, 4, "ring")])
def test_rs_one_row_per_shard(ub, tp, T, order):
    """T == tp: every shard is one row; with 64 ranks the ring has 63 hops."""
    rng = np.random.default_rng(tp * 7 + T)
    H, K = 64, 64 * tp
    a = wl.normal_bits(rng, (T, K))
    w = wl.normal_bits(rng, (K, H), 0.05)
    print(f"[edge rs] tp={tp} T={T} {order}", flush=True)
    reg = gu.Registration(ub, T, H, tp)
    try:
        reg.set_T(T)
        for atomic in (False, True):
            out = gu.canary((T + 2, H))
            ub.ub_gemm_rs_chunked(reg.h, gu.dev(a), K, K, gu.dev(w), H, out, H,
                                  ub.make_cfg("ring_exchange", 1, atomic_gemm=atomic, reduce_order=order))
            torch.cuda.synchronize()
            oh = gu.host(out)
            if order == "ring":
                want, _ = og.rs_rows_ring(np.arange(T), a, w, T, tp)
            else:
                want, _ = og.rs_rows(a, w, tp)
            # ring: a partial that differs in its last bit changes every later hop, so fewer
            # results are bit-equal; the bound is the check
            gu.check_rs_close(oh[:T], want, a, w, tp, f"edge rs tp={tp} T={T} {order} atomic={atomic}",
                              min_equal=0.2 if order == "ring" else 0.9, ring=order == "ring")
            assert np.all(oh[T:] == gu.CANARY)
            parts = gu.host(reg.ws_t)[: tp * T * H].reshape(tp, T, H)
            ks = K // tp
            for s in (0, tp - 1):
                gu.check_close(parts[s], og.rs_rows(a, w[:, :], tp)[1][s], a[:, s * ks:(s + 1) * ks],
                               w[s * ks:(s + 1) * ks], f"partial {s}")
    finally:
        reg.close()


def test_gqa_at_capacity_sampled(ub):
    """The largest registration of the workloads (capacity 32768, hidden 8192) at
    T == capacity in the device-side loop: sampled rows against the oracle."""
    w = wl.gqa_bulk()
    ra, rw, _ = w.seeds()
    T = w.capacity
    a = wl.activations(w, T, ra)
    wt = wl.weights(w, rw)
    reg = gu.Registration(ub, w.capacity, w.hidden, w.tp, workspace=False, pad_rows=4)
    rng = np.random.default_rng(81)
    try:
        reg.set_T(T)
        reg.fill(a)
        c = gu.canary((w.capacity + 4, w.n_cols))
        ub.ub_gemm_ag_chunked(reg.h, gu.dev(wt), w.n_cols, w.n_cols, c, w.n_cols,
                              ub.make_cfg(w.method, w.num_splits, atomic_gemm=True))
        torch.cuda.synchronize()
        ch = gu.host(c)
        assert np.all(ch[T:] == gu.CANARY)
        rows = np.array(sorted(set(rng.integers(0, T, size=12).tolist()) | {0, T - 1, T // 2}))
        gu.check_close(ch[rows], og.ag_rows(a[rows], wt), a[rows], wt, "gqa at capacity")
    finally:
        reg.close()
