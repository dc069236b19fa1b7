"""GPU parity of the reduce-scatter-side chunked GEMM (ub_gemm_rs_chunked) and of the
partial-sum reduction (ub_reduce_partials) against the oracle."""

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


def _run_rs(ub, reg, a_t, k, w_t, cfg, stream=None, extra_rows=8):
    H = reg.hidden
    out = gu.canary((reg.capacity + extra_rows, H))
    ub.ub_gemm_rs_chunked(reg.h, a_t, k, k, w_t, H, out, H, cfg, stream)
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


def test_tiny_rs_matches_oracle(ub):
    w = wl.tiny_rs()
    ra, rw, _ = w.seeds()
    T = 256
    a = wl.activations(w, T, ra)
    wt = wl.weights(w, rw)
    print(f"[tiny_rs] T={T} K={w.k} H={w.hidden} tp={w.tp}", flush=True)
    reg = gu.Registration(ub, w.capacity, w.hidden, w.tp, pad_rows=16)
    try:
        reg.set_T(T)
        out = _run_rs(ub, reg, gu.dev(a), w.k, gu.dev(wt), ub.make_cfg(w.method, w.num_splits))
        ref, parts = _oracle_rs(w.capacity, w.hidden, w.tp, a, wt, op.OverlapCfg(method=w.method))
        print(gu.check_rs_close(out[:T], ref, a, wt, w.tp, "tiny_rs"))
        ws = gu.host(reg.ws_t)
        ks = w.k // w.tp
        for s in range(w.tp):
            slot = ws[s * T * w.hidden:(s + 1) * T * w.hidden].reshape(T, w.hidden)
            gu.check_close(slot, parts[s], a[:, s * ks:(s + 1) * ks], wt[s * ks:(s + 1) * ks],
                           f"tiny_rs partial {s}")
        assert np.all(ws[w.tp * T * w.hidden:] == gu.CANARY)  # workspace tail untouched
        assert np.all(out[T:] == gu.CANARY)
        shards = og.shards(out, T, w.hidden, w.tp)
        assert np.array_equal(np.concatenate(shards), out[:T])
    finally:
        reg.close()


@pytest.mark.parametrize("cap,H,K,T,tp,method,ns", [
    (512, 256, 256, 256, 2, "ring_exchange", 2),
    (1024, 512, 1024, 296, 8, "pipeline", 4),       # 8 slices of 128, ragged chunks
    (256, 64, 1024, 96, 4, "bulk", 5),
    (64, 128, 512, 64, 1, "pipeline", 2),            # tp = 1: a plain GEMM
    (768, 136, 768, 294, 6, "ring_exchange", 6),     # tp = 6: the run-time slot count
])
def test_integer_inputs_bit_exact(ub, cap, H, K, T, tp, method, ns):
    rng = np.random.default_rng(cap + H + K + T)
    a = wl.integer_bits(rng, (T, K))
    wt = wl.integer_bits(rng, (K, H))
    print(f"[int_rs] cap={cap} H={H} K={K} T={T} tp={tp} {method} ns={ns}", flush=True)
    reg = gu.Registration(ub, cap, H, tp, pad_rows=8)
    try:
        reg.set_T(T)
        ref, parts = _oracle_rs(cap, H, tp, a, wt, op.OverlapCfg(method=method, num_splits=ns))
        for atomic in (False, True):
            reg.ws_t.fill_(gu.CANARY)
            out = _run_rs(ub, reg, gu.dev(a), K, gu.dev(wt), ub.make_cfg(method, ns, atomic_gemm=atomic))
            assert np.array_equal(out[:T], ref), atomic
            ws = gu.host(reg.ws_t)
            assert np.array_equal(ws[: tp * T * H].reshape(tp, T, H), parts)
            assert np.all(ws[tp * T * H:] == gu.CANARY)
            assert np.all(out[T:] == gu.CANARY)
    finally:
        reg.close()


@pytest.mark.parametrize("tile", gu.BF16_TILES)
def test_every_tile_shape_rs(ub, tile):
    """Each GEMM tile shape, forced, on the slice GEMMs: integer inputs bit-exact against
    the oracle (partials and output), ragged rows and chunks."""
    rng = np.random.default_rng(22)
    cap, H, K, T, tp = 1024, 264, 2048, 600, 8
    a = wl.integer_bits(rng, (T, K))
    wt = wl.integer_bits(rng, (K, H))
    print(f"[rs tile {tile}] cap={cap} H={H} K={K} T={T}", flush=True)
    reg = gu.Registration(ub, cap, H, tp, pad_rows=8)
    gu.force_tile(ub, reg.h, tile)
    try:
        reg.set_T(T)
        ref, parts = _oracle_rs(cap, H, tp, a, wt, op.OverlapCfg(method="pipeline", num_splits=3))
        for atomic in (False, True):
            reg.ws_t.fill_(gu.CANARY)
            out = _run_rs(ub, reg, gu.dev(a), K, gu.dev(wt), ub.make_cfg("pipeline", 3, atomic_gemm=atomic))
            assert np.array_equal(out[:T], ref), atomic
            ws = gu.host(reg.ws_t)
            assert np.array_equal(ws[: tp * T * H].reshape(tp, T, H), parts)
            assert np.all(ws[tp * T * H:] == gu.CANARY)
            assert np.all(out[T:] == gu.CANARY)
    finally:
        reg.close()


def test_strided_output_rows(ub):
    """ldo > H: the reduction writes only the first H columns of each output row, and the
    values equal those of the packed output."""
    rng = np.random.default_rng(23)
    T, H, K, tp, ldo = 200, 200, 1024, 8, 232
    a = gu.dev(wl.normal_bits(rng, (T, K)))
    wt = gu.dev(wl.normal_bits(rng, (K, H), 0.02))
    reg = gu.Registration(ub, 256, H, tp)
    try:
        reg.set_T(T)
        ref = _run_rs(ub, reg, a, K, wt, ub.make_cfg("pipeline", 3))[:T]
        for atomic in (False, True):
            out = gu.canary((T + 3, ldo))
            ub.ub_gemm_rs_chunked(reg.h, a, K, K, wt, H, out, ldo, ub.make_cfg("pipeline", 3, atomic_gemm=atomic))
            torch.cuda.synchronize()
            oh = gu.host(out)
            assert np.array_equal(oh[:T, :H], ref), atomic
            assert np.all(oh[:T, H:] == gu.CANARY) and np.all(oh[T:] == gu.CANARY)
            out2 = gu.canary((T, ldo))
            ub.ub_reduce_partials(reg.h, out2, ldo)
            torch.cuda.synchronize()
            oh2 = gu.host(out2)
            assert np.array_equal(oh2[:, :H], ref) and np.all(oh2[:, H:] == gu.CANARY)
    finally:
        reg.close()


def test_closed_form_fc2_ones(ub):
    """K = 14336 in 8 slices: every partial is 1792 and every output 14336, exactly."""
    T, H, K, tp = 64, 256, 14336, 8
    reg = gu.Registration(ub, 128, H, tp)
    try:
        reg.set_T(T)
        out = _run_rs(ub, reg, gu.dev(wl.const_bits((T, K), 1.0)), K,
                      gu.dev(wl.const_bits((K, H), 1.0)), ub.make_cfg("pipeline", 4))
        assert np.all(out[:T] == wl.const_bits((1,), 14336.0)[0])
        ws = gu.host(reg.ws_t)[: tp * T * H]
        assert np.all(ws == wl.const_bits((1,), 1792.0)[0])
    finally:
        reg.close()


def test_bit_identical_across_schedules(ub):
    rng = np.random.default_rng(5)
    T, H, K, tp = 232, 128, 1024, 4
    a = gu.dev(wl.normal_bits(rng, (T, K)))
    wt = gu.dev(wl.normal_bits(rng, (K, H), 0.02))
    reg = gu.Registration(ub, 512, H, tp)
    try:
        reg.set_T(T)
        ref = _run_rs(ub, reg, a, K, wt, ub.make_cfg("pipeline", 1))[:T]
        ref_ws = gu.host(reg.ws_t)[: tp * T * H].copy()
        for method in ("ring_exchange", "pipeline", "bulk"):
            for ns in (1, 2, 3, 4, 7):
                for nms in (1, 2, 3):
                    for rank in (0, 3):
                        for atomic in (False, True):
                            cfg = ub.make_cfg(method, ns, nms, atomic_gemm=atomic, rank=rank)
                            got = _run_rs(ub, reg, a, K, wt, cfg)[:T]
                            assert np.array_equal(got, ref), (method, ns, nms, rank, atomic)
                            assert np.array_equal(gu.host(reg.ws_t)[: tp * T * H], ref_ws)
    finally:
        reg.close()


def _seeded_partials(rng, tp, T, H):
    """bf16 partials over a few binades, both signs, some exact zeros and cancelling pairs:
    the reduction's input, generated here rather than by a GEMM."""
    x = rng.standard_normal((tp, T, H)) * np.exp2(rng.integers(-6, 7, size=(tp, T, H)))
    x[rng.random((tp, T, H)) < 0.02] = 0.0
    x[1] = np.where(rng.random((T, H)) < 0.05, -x[0], x[1])
    from oracle import bf16 as ob
    return ob.encode_rne(x)


def test_reduce_partials_alone_matches(ub):
    """ub_reduce_partials reproduces the reduce-scatter call's own sum, and, on seeded
    partials written into the workspace by the test, matches the oracle: ascending order
    within the fp32-sum bound (bit-equal where that sum is exact), ring order bit for bit."""
    from oracle import bf16 as ob
    rng = np.random.default_rng(6)
    T, H, K, tp = 296, 256, 2048, 8
    a = wl.normal_bits(rng, (T, K))
    wt = wl.normal_bits(rng, (K, H), 0.02)
    reg = gu.Registration(ub, 512, H, tp)
    try:
        reg.set_T(T)
        out = _run_rs(ub, reg, gu.dev(a), K, gu.dev(wt), ub.make_cfg("pipeline", 4))
        out2 = gu.canary((T + 4, H))
        ub.ub_reduce_partials(reg.h, out2, H)
        torch.cuda.synchronize()
        out2 = gu.host(out2)
        assert np.array_equal(out2[:T], out[:T])
        assert np.all(out2[T:] == gu.CANARY)
        # the reduction alone on partials generated here
        parts = _seeded_partials(rng, tp, T, H)
        reg.ws_t[: tp * T * H].copy_(gu.dev(parts).reshape(-1))
        dec = [ob.decode(parts[s]) for s in range(tp)]
        exact = ob.encode_rne(og.exact_sum(dec) + 0.0)
        for order in ("ascending", "ring"):
            o3 = gu.canary((T + 4, H))
            ub.ub_reduce_partials(reg.h, o3, H, order)
            torch.cuda.synchronize()
            o3 = gu.host(o3)
            assert np.all(o3[T:] == gu.CANARY)
            if order == "ring":
                assert np.array_equal(o3[:T], og.ring_sum(dec, 0, T, tp))
            else:
                gap = np.abs(ob.decode(o3[:T]) - ob.decode(exact))
                bound = ob.ulp(exact) + tp * 2.0 ** -24 * np.sum(np.abs(np.array(dec)), axis=0)
                assert np.all(gap <= bound)
                assert np.mean(o3[:T] == exact) >= 0.99
        assert bool((reg.ws_t[tp * T * H:] == gu.CANARY).all().item())
    finally:
        reg.close()


def test_fc2_full_size_sampled(ub):
    """The MLP fc2 workload (capacity 16384, hidden 4096, K 14336 in 8 slices, pipeline
    with 4 chunks) at each T of its sweep, on one registration; sampled rows vs the
    oracle, workspace and output tails untouched."""
    w = wl.fc2()
    ra, rw, _ = w.seeds()
    a_all = wl.activations(w, w.capacity, ra)
    wt = wl.weights(w, rw)
    a_t, w_t = gu.dev(a_all), gu.dev(wt)
    H, tp = w.hidden, w.tp
    reg = gu.Registration(ub, w.capacity, H, tp, pad_rows=8)
    rng = np.random.default_rng(7)
    cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams)
    try:
        out = gu.canary((w.capacity + 8, H))
        for T in wl.FC2_TOKENS:
            print(f"[fc2] T={T}", flush=True)
            reg.set_T(T)
            out.fill_(gu.CANARY)
            reg.ws_t.fill_(gu.CANARY)
            ub.ub_gemm_rs_chunked(reg.h, a_t, w.k, w.k, w_t, H, out, H, cfg)
            torch.cuda.synchronize()
            oh = gu.host(out)
            rows = set(rng.integers(0, T, size=24).tolist()) | {0, T - 1}
            for c in range(1, w.num_splits):
                rows |= {(c * T) // w.num_splits - 1, (c * T) // w.num_splits}
            for r in range(1, tp):
                rows |= {r * T // tp - 1, r * T // tp}  # shard boundaries
            rows = np.array(sorted(rows))
            ref, _ = og.rs_rows(a_all[rows], wt, tp)
            gu.check_rs_close(oh[rows], ref, a_all[rows], wt, tp, f"fc2 T={T}")
            assert np.all(oh[T:] == gu.CANARY)
            tail = reg.ws_t[tp * T * H:]
            assert bool((tail == gu.CANARY).all().item())
    finally:
        reg.close()


# ---- ring-order reduce-scatter (reduce_order="ring") -------------------------------------

def _gpu_parts(reg, tp, T, H):
    return gu.host(reg.ws_t)[: tp * T * H].reshape(tp, T, H)


def test_ring_reduce_schedule_identical(ub):
    """Ring order end to end: every schedule (chunking, streams, rank, device-side loop)
    gives the same bits as the first, leaves the same partials in the workspace as the
    ascending order does, and differs from the ascending result on random data; the
    ring sum itself is pinned bit for bit on seeded partials in
    test_reduce_partials_alone_matches, and against the oracle end to end on integer
    inputs below."""
    rng = np.random.default_rng(41)
    T, H, K, tp = 240, 136, 1024, 8
    a = gu.dev(wl.normal_bits(rng, (T, K)))
    wt = gu.dev(wl.normal_bits(rng, (K, H), 0.02))
    reg = gu.Registration(ub, 512, H, tp)
    try:
        reg.set_T(T)
        asc = _run_rs(ub, reg, a, K, wt, ub.make_cfg("pipeline", 1))[:T]
        parts = _gpu_parts(reg, tp, T, H).copy()
        ref = _run_rs(ub, reg, a, K, wt, ub.make_cfg("pipeline", 1, reduce_order="ring"))[:T]
        assert not np.array_equal(ref, asc)
        for method in ("ring_exchange", "pipeline", "bulk"):
            for ns in (1, 3, 4):
                for rank in (0, 5):
                    for atomic in (False, True):
                        cfg = ub.make_cfg(method, ns, 3, atomic_gemm=atomic, rank=rank,
                                          reduce_order="ring")
                        got = _run_rs(ub, reg, a, K, wt, cfg)
                        assert np.array_equal(got[:T], ref), (method, ns, rank, atomic)
                        assert np.all(got[T:] == gu.CANARY)
                        assert np.array_equal(_gpu_parts(reg, tp, T, H), parts)
        out2 = gu.canary((T + 2, H))
        ub.ub_reduce_partials(reg.h, out2, H, "ring")
        torch.cuda.synchronize()
        o2 = gu.host(out2)
        assert np.array_equal(o2[:T], ref) and np.all(o2[T:] == gu.CANARY)
    finally:
        reg.close()


@pytest.mark.parametrize("tp,T,method,ns", [(8, 296, "ring_exchange", 8), (6, 294, "pipeline", 4),
                                            (2, 64, "bulk", 3), (1, 40, "bulk", 2)])
def test_ring_reduce_integer_inputs_end_to_end(ub, tp, T, method, ns):
    """Integer inputs: GPU partials are exact, so the whole ring reduce-scatter equals the
    oracle's bit for bit (hops round: partial values exceed 256)."""
    rng = np.random.default_rng(42 + tp)
    H, K = 128, 512 * tp
    a = wl.integer_bits(rng, (T, K))
    wt = wl.integer_bits(rng, (K, H))
    cap = T + 8 * tp
    reg = gu.Registration(ub, cap, H, tp, pad_rows=8)
    try:
        reg.set_T(T)
        ref, parts = _oracle_rs(cap, H, tp, a, wt, op.OverlapCfg(method=method, num_splits=ns,
                                                                 reduce_order="ring"))
        for atomic in (False, True):
            out = _run_rs(ub, reg, gu.dev(a), K, gu.dev(wt),
                          ub.make_cfg(method, ns, atomic_gemm=atomic, reduce_order="ring"))
            assert np.array_equal(out[:T], ref), atomic
            assert np.array_equal(_gpu_parts(reg, tp, T, H), parts)
    finally:
        reg.close()


def test_ring_reduce_fc2_full_size_sampled(ub):
    """fc2 (capacity 16384, hidden 4096, K 14336 in 8 slices) at its largest T in ring
    order: sampled rows (every shard boundary) against the oracle's ring reduce-scatter of
    the same rows within the ring bound, and the partials against the oracle's within the
    gate."""
    w = wl.fc2()
    ra, rw, _ = w.seeds()
    T = wl.FC2_TOKENS[-1]
    a_all = wl.activations(w, T, ra)
    wt = wl.weights(w, rw)
    H, tp = w.hidden, w.tp
    reg = gu.Registration(ub, w.capacity, H, tp, pad_rows=8)
    rng = np.random.default_rng(43)
    try:
        reg.set_T(T)
        out = gu.canary((w.capacity + 8, H))
        cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, atomic_gemm=True,
                          reduce_order="ring")
        print(f"[fc2 ring] T={T}", flush=True)
        ub.ub_gemm_rs_chunked(reg.h, gu.dev(a_all), w.k, w.k, gu.dev(wt), H, out, H, cfg)
        torch.cuda.synchronize()
        rows = set(rng.integers(0, T, size=16).tolist()) | {0, T - 1}
        for r in range(1, tp):
            rows |= {r * T // tp - 1, r * T // tp}
        rows = np.array(sorted(rows))
        ws = reg.ws_t[: tp * T * H].view(tp, T, H)
        parts = [gu.host(ws[s][torch.as_tensor(rows, device=ws.device)]) for s in range(tp)]
        oh = gu.host(out)
        ref, oparts = og.rs_rows_ring(rows, a_all[rows], wt, T, tp)
        gu.check_rs_close(oh[rows], ref, a_all[rows], wt, tp, "fc2 ring", min_equal=0.2, ring=True)
        ks = w.k // tp
        for s in range(tp):
            gu.check_close(parts[s], oparts[s], a_all[rows][:, s * ks:(s + 1) * ks],
                           wt[s * ks:(s + 1) * ks], f"fc2 ring partial {s}")
        assert np.all(oh[T:] == gu.CANARY)
    finally:
        reg.close()


@pytest.mark.parametrize("ks", (40, 72))
@pytest.mark.parametrize("fuse", (False, True))
def test_slice_width_not_multiple_of_k_step(ub, ks, fuse):
    """K / tp a multiple of 8 but not of the kernel's 32-deep k-step: each slice's last
    step masks the A chunks that belong to the next slice.  Integer inputs: partials and
    output bit-exact against the oracle for every tile shape, both schedules and both
    summation orders; the counters of the fused sum end at zero."""
    rng = np.random.default_rng(150 + ks)
    cap, H, T, tp = 1024, 264, 600, 8
    K = tp * ks
    a = wl.integer_bits(rng, (T, K))
    wt = wl.integer_bits(rng, (K, H))
    reg = gu.Registration(ub, cap, H, tp, pad_rows=8)
    try:
        reg.set_T(T)
        for order in ("ascending", "ring"):
            ref, parts = _oracle_rs(cap, H, tp, a, wt, op.OverlapCfg(method="pipeline", num_splits=3,
                                                                     reduce_order=order))
            for tile in gu.BF16_TILES:
                gu.force_tile(ub, reg.h, tile)
                for atomic in (False, True):
                    print(f"[slice tail] ks={ks} fuse={fuse} {order} {tile} atomic={atomic}", flush=True)
                    reg.ws_t.fill_(gu.CANARY)
                    out = _run_rs(ub, reg, gu.dev(a), K, gu.dev(wt),
                                  ub.make_cfg("pipeline", 3, atomic_gemm=atomic, reduce_order=order,
                                              fuse_reduce=fuse))
                    assert np.array_equal(out[:T], ref), (order, tile, atomic)
                    ws = gu.host(reg.ws_t)
                    assert np.array_equal(ws[: tp * T * H].reshape(tp, T, H), parts)
                    assert np.all(out[T:] == gu.CANARY)
        assert reg.counters_clean()
    finally:
        reg.close()


# ---- pipelined device-side reduce-scatter (rs_pieces) ------------------------------------

def _rs_piece_count(T, P):
    """Pieces the library cuts T rows into for P requested: cuts on multiples of 1280 rows
    nearest to p T / P, strictly increasing and inside (0, T)."""
    cuts = [0]
    for p in range(1, P):
        c = (T * p // P + 640) // 1280 * 1280
        if cuts[-1] < c < T:
            cuts.append(c)
    return len(cuts)


@pytest.mark.parametrize("ring", (False, True))
def test_pipelined_device_loop_pieces_bit_identical(ub, ring):
    """The device-side loop in 1..8 row pieces (each piece's reduction on a worker stream,
    overlapping the next piece's GEMMs): output bit-identical to one launch + one
    reduction and to the host loop; integer inputs equal the oracle bit for bit; plan
    record counts the pieces and the GEMM dispatches."""
    rng = np.random.default_rng(61 + ring)
    cap, H, K, tp = 8192, 512, 2048, 8
    for T, ints in ((7680, True), (6136, False)):
        a = (wl.integer_bits if ints else wl.normal_bits)(rng, (T, K))
        wt = wl.integer_bits(rng, (K, H)) if ints else wl.normal_bits(rng, (K, H), 0.02)
        a_t, w_t = gu.dev(a), gu.dev(wt)
        reg = gu.Registration(ub, cap, H, tp, pad_rows=8)
        try:
            reg.set_T(T)
            order = "ring" if ring else "ascending"
            base = ub.make_cfg("pipeline", 4, atomic_gemm=True, reduce_order=order)
            ub.ub_debug_set(reg.h, "rs_pieces", 1)
            ref = _run_rs(ub, reg, a_t, K, w_t, base)
            assert ub.ub_debug_plan(reg.h)["rs_pieces"] == 0
            if ints:
                o, _ = _oracle_rs(cap, H, tp, a, wt, op.OverlapCfg(method="pipeline", num_splits=4,
                                                                   reduce_order=order))
                assert np.array_equal(ref[:T], o)
            for pieces in (2, 3, 4, 8):
                print(f"[rs pieces] T={T} ring={ring} pieces={pieces}", flush=True)
                ub.ub_debug_set(reg.h, "rs_pieces", pieces)
                got = _run_rs(ub, reg, a_t, K, w_t, base)
                assert np.array_equal(got, ref), pieces
                plan = ub.ub_debug_plan(reg.h)
                assert plan["rs_pieces"] == _rs_piece_count(T, pieces), plan
                assert plan["dispatches"] >= plan["rs_pieces"]
            ub.ub_debug_set(reg.h, "rs_pieces", 0)
            host = _run_rs(ub, reg, a_t, K, w_t, ub.make_cfg("pipeline", 4, reduce_order=order))
            assert np.array_equal(host, ref)
            assert reg.counters_clean()
        finally:
            reg.close()


def test_pipelined_fc2_full_size_sampled(ub):
    """fc2 (capacity 16384, hidden 4096, K 14336 in 8 slices) in the device-side loop with
    4 row pieces at T = 16384 and 12280: bit-identical to the unpipelined call, sampled
    rows against the oracle."""
    w = wl.fc2()
    ra, rw, _ = w.seeds()
    a_all = wl.activations(w, w.capacity, ra)
    wt = wl.weights(w, rw)
    a_t, w_t = gu.dev(a_all), gu.dev(wt)
    H, tp = w.hidden, w.tp
    reg = gu.Registration(ub, w.capacity, H, tp, pad_rows=8)
    rng = np.random.default_rng(17)
    cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, atomic_gemm=True)
    try:
        out = gu.canary((w.capacity + 8, H))
        for T in (16384, 12280):
            print(f"[fc2 pieces] T={T}", flush=True)
            reg.set_T(T)
            outs = []
            for pieces in (1, 4):
                ub.ub_debug_set(reg.h, "rs_pieces", pieces)
                out.fill_(gu.CANARY)
                ub.ub_gemm_rs_chunked(reg.h, a_t, w.k, w.k, w_t, H, out, H, cfg)
                torch.cuda.synchronize()
                outs.append(gu.host(out))
            assert np.array_equal(outs[0], outs[1])
            rows = np.array(sorted(set(rng.integers(0, T, size=24).tolist()) |
                                   {0, T - 1, 3839, 3840, 7679, 7680, 11519, 11520} - {r for r in range(T, 16384)}))
            ref, _ = og.rs_rows(a_all[rows], wt, tp)
            gu.check_rs_close(outs[1][rows], ref, a_all[rows], wt, tp, f"fc2 pieces T={T}")
            assert np.all(outs[1][T:] == gu.CANARY)
    finally:
        ub.ub_debug_set(reg.h, "rs_pieces", 0)
        reg.close()
