"""GPU parity of the FP8 (E4M3) path against the oracle (oracle.fp8): ub_quantize_in,
ub_quantize_e4m3, ub_gemm_ag_chunked_fp8 and ub_gemm_rs_chunked_fp8."""

import numpy as np
import pytest
import torch

from chunked_tp_overlap_amd import workloads as wl
from oracle import bf16 as ob
from oracle import fp8 as of
from oracle import plan as op
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CANARY8 = 0x7F  # an E4M3 NaN: a read of it would poison the result


@pytest.fixture(scope="module")
def ub():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import chunked_tp_overlap_amd.ub as m
    return m


class Fp8Reg:
    def __init__(self, ub, capacity, hidden, tp, pad_rows=8):
        self.ub, self.capacity, self.hidden = ub, capacity, hidden
        self.buf = torch.full(((capacity + pad_rows) * hidden,), CANARY8, dtype=torch.uint8, device="cuda")
        self.h = ub.ub_init(capacity, hidden, tp, ub.UB_DTYPE_FP8_E4M3, self.buf, capacity * hidden)

    def host(self):
        return self.buf.cpu().numpy()

    def close(self):
        self.ub.ub_destroy(self.h)


def _dev8(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).cuda()


def _mixed_bf16(rng, shape):
    """bf16 values over a wide range, with zeros, signed zeros, infinities and values at
    the E4M3 limits (NaN is covered separately)."""
    x = rng.standard_normal(shape) * np.exp2(rng.integers(-14, 12, size=shape))
    flat = x.ravel()
    specials = [0.0, -0.0, np.inf, -np.inf, 448.0, -448.0, 464.0, 479.9, 2.0 ** -6,
                2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, -(2.0 ** -12), 1.0625, 1.1875]
    idx = rng.choice(flat.size, size=len(specials) * 8, replace=False)
    flat[idx] = np.repeat(specials, 8)
    return ob.encode_rne(flat.reshape(shape))


@pytest.mark.parametrize("scale", [1.0, 0.25, 37.5, 1.3, 448.0 / 11.7])
def test_quantize_bit_exact(ub, scale):
    rng = np.random.default_rng(71)
    cap, H, T, tp = 512, 256, 400, 8
    x = _mixed_bf16(rng, (T, H))
    reg = Fp8Reg(ub, cap, H, tp)
    try:
        ub.ub_set_active_shape(reg.h, (T, H))
        r0, rows = 50, 300
        print(f"[quantize] scale={scale}", flush=True)
        ub.ub_quantize_in(reg.h, gu.dev(x[r0:r0 + rows]), rows, r0, scale)
        torch.cuda.synchronize()
        got = reg.host()
        want = of.quantize(x[r0:r0 + rows], np.float32(scale))
        assert np.array_equal(got[r0 * H:(r0 + rows) * H].reshape(rows, H), want)
        assert np.all(got[: r0 * H] == CANARY8) and np.all(got[(r0 + rows) * H:] == CANARY8)
    finally:
        reg.close()


def test_quantize_nan(ub):
    reg = Fp8Reg(ub, 16, 16, 1)
    try:
        x = np.full((1, 16), 0x7FC0, np.uint16)  # bf16 quiet NaN
        ub.ub_quantize_in(reg.h, gu.dev(x), 1, 3, 2.0)
        torch.cuda.synchronize()
        assert np.all((reg.host()[3 * 16:4 * 16] & 0x7F) == 0x7F)
    finally:
        reg.close()


def _int_codes(rng, shape, lo=-8, hi=8):
    return of.encode(rng.integers(lo, hi + 1, size=shape).astype(np.float64))


def _gemm(ub, reg, w_codes, n, sa, sw, cfg, ldc=None):
    ldc = ldc or n
    c = gu.canary((reg.capacity + 4, ldc))
    ub.ub_gemm_ag_chunked_fp8(reg.h, _dev8(w_codes), n, w_codes.shape[1], sa, sw, c, ldc, cfg)
    torch.cuda.synchronize()
    return gu.host(c)


@pytest.mark.parametrize("tile", ["256x256", "128x256", "256x192"])
def test_gemm_integer_bit_exact_every_schedule(ub, tile):
    """Small-integer codes, power-of-two scales: every partial sum is exact in fp32, so
    GPU == oracle bit for bit, for every chunking (up to a 64-unit device-side loop), stream
    count, rank, aggregate setting, and every tile shape."""
    rng = np.random.default_rng(72)
    cap, H, N, T, tp = 1024, 512, 264, 600, 8
    a = _int_codes(rng, (T, H))
    w = _int_codes(rng, (N, H))
    sa, sw = 2.0 ** -3, 2.0 ** -5
    reg = Fp8Reg(ub, cap, H, tp)
    gu.force_tile(ub, reg.h, tile)
    try:
        ub.ub_set_active_shape(reg.h, (T, H))
        ub.ub_copy_in(reg.h, _dev8(a), T, 0)
        units = op.build(T, tp, op.OverlapCfg(method="bulk"), "ag")
        want, _ = of.ag_chunked_fp8(T, a.ravel(), H, w, N, sa, sw, units)
        for method, ns, nms, agg, rank, atomic in [("ring_exchange", 1, 3, False, 0, False),
                                                  ("ring_exchange", 1, 3, False, 5, True),
                                                  ("ring_exchange", 1, 2, True, 3, True),
                                                  ("pipeline", 7, 3, False, 0, False),
                                                  ("bulk", 3, 1, True, 0, True),
                                                  ("pipeline", 64, 3, False, 0, True)]:
            cfg = ub.make_cfg(method, ns, nms, agg, atomic, rank=rank)
            got = _gemm(ub, reg, w, N, sa, sw, cfg)
            assert np.array_equal(got[:T], want), (tile, method, ns, nms, agg, rank, atomic)
            assert np.all(got[T:] == gu.CANARY)
        assert np.all(reg.host()[T * H:] == CANARY8)  # the UB tail was only a canary
    finally:
        reg.close()


# How the f8f6f4 MFMA sums (pinned by test_mfma_block_sum_model below): within one
# instruction, i.e. one 64-code block of k, the products are added at fixed point aligned
# to the block's largest |product| 2**e (e = floor(log2)), and the bits below 2**(e - 14)
# are dropped; between blocks the sum is an fp32 accumulator.  So each nonzero product of
# a block is off by less than 2**(e - 14), and each block adds one fp32 rounding.
def mfma8_block_err(A, W):
    """Bound on the in-block loss of the FP8 GEMM A [T, K] x W [N, K]^T (decoded values)."""
    T, K = A.shape
    out = np.zeros((T, W.shape[0]))
    for b in range(0, K, 64):
        P = np.abs(A[:, None, b:b + 64] * W[None, :, b:b + 64])
        m = P.max(axis=2)
        e = np.floor(np.log2(np.where(m > 0, m, 1.0)))
        out += np.where(m > 0, (P > 0).sum(axis=2) * np.exp2(e - 14), 0.0)
    return out


def fp8_slice_err(a_codes, w_codes, scale):
    """Accumulation error bound of an FP8 GEMM (before the bf16 rounding), scaled: the
    in-block loss plus one fp32 rounding per block and two for the scale multiply."""
    A, W = of.decode(a_codes), of.decode(w_codes)
    K = A.shape[1]
    absdot = np.abs(A) @ np.abs(W).T
    return (mfma8_block_err(A, W) + (K // 64 + 2) * 2.0 ** -24 * (absdot + mfma8_block_err(A, W))) * scale


def _check_tol(got, want, a_codes, w_codes, sa, sw, what, min_equal=0.98):
    A = of.decode(a_codes)
    W = of.decode(w_codes)
    g = ob.decode(got)
    o = ob.decode(want)
    absdot = (np.abs(A) @ np.abs(W).T) * sa * sw
    tight = np.maximum(ob.ulp(got), ob.ulp(want)) + fp8_slice_err(a_codes, w_codes, sa * sw)
    gate = 4e-3 * np.outer(np.linalg.norm(A, axis=1), np.linalg.norm(W, axis=1)) * sa * sw
    err = np.abs(g - o)
    assert np.all(err <= gate), f"{what}: gate"
    if not np.all(err <= tight):
        bad = np.argwhere(err > tight)[:6]
        exact = (A @ W.T) * sa * sw
        info = [(tuple(int(x) for x in ij), hex(int(got[tuple(ij)])), hex(int(want[tuple(ij)])),
                 float(g[tuple(ij)]), float(o[tuple(ij)]), float(exact[tuple(ij)]),
                 float(tight[tuple(ij)]), float(absdot[tuple(ij)])) for ij in bad]
        raise AssertionError(f"{what}: tight bound at {int(np.sum(err > tight))} elements: "
                             f"(index, got, want, got value, want value, exact, bound, sum|ab|) {info}")
    eq = np.mean(got == want)
    assert eq >= min_equal, f"{what}: only {eq:.4f} bit-equal"
    return float(eq)


def test_gemm_random_codes_within_tolerance_and_schedule_identical(ub):
    rng = np.random.default_rng(73)
    cap, H, N, T, tp = 512, 1024, 200, 296, 8
    a = rng.integers(0, 256, size=(T, H)).astype(np.uint8)
    w = rng.integers(0, 256, size=(N, H)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38
    w[(w & 0x7F) == 0x7F] = 0x38
    sa, sw = 0.37, 0.0021
    reg = Fp8Reg(ub, cap, H, tp)
    try:
        ub.ub_set_active_shape(reg.h, (T, H))
        ub.ub_copy_in(reg.h, _dev8(a), T, 0)
        ref = _gemm(ub, reg, w, N, sa, sw, ub.make_cfg("bulk", 1))[:T]
        want = of.ag_rows_fp8(a, w, N, np.float32(sa) * np.float32(sw), 1.0)
        # codes over all 17 binades of E4M3: products span 2**35 and sums cancel, so more
        # results sit within the fp32 accumulation error of a bf16 rounding boundary
        eq = _check_tol(ref, want, a, w, sa, sw, "fp8 random", min_equal=0.95)
        print(f"[fp8 random] bit-equal {eq:.4f}")
        for method in ("ring_exchange", "pipeline", "bulk"):
            for ns in (2, 5):
                for atomic in (False, True):
                    got = _gemm(ub, reg, w, N, sa, sw, ub.make_cfg(method, ns, 3, False, atomic, rank=2))
                    assert np.array_equal(got[:T], ref), (method, ns, atomic)
    finally:
        reg.close()


def test_fp8_qkv_full_size_sampled(ub):
    """The QKV workload quantized: activations [8192, 4096] through ub_quantize_in with a
    per-tensor scale 448 / amax, weights [1536, 4096] quantized by the oracle; the
    device-side chunk loop over 8 ring chunks at T = 8192 and T = 5000; sampled rows
    (every chunk boundary) against the oracle within tolerance."""
    w = wl.qkv()
    ra, rw, _ = w.seeds()
    H, N, tp = w.hidden, w.n_cols, w.tp
    x = wl.activations(w, w.capacity, ra)
    wt = wl.weights(w, rw)
    amax_x = float(np.max(np.abs(ob.decode(x))))
    amax_w = float(np.max(np.abs(ob.decode(wt))))
    sx, swq = np.float32(448.0 / amax_x), np.float32(448.0 / amax_w)
    w_codes = of.quantize(np.ascontiguousarray(wt.T), swq)  # [N, K]
    reg = Fp8Reg(ub, w.capacity, H, tp)
    rng = np.random.default_rng(74)
    try:
        for T in (w.capacity, 5000):
            print(f"[fp8 qkv] T={T}", flush=True)
            ub.ub_set_active_shape(reg.h, (T, H))
            ub.ub_quantize_in(reg.h, gu.dev(x[:T]), T, 0, float(sx))
            cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, atomic_gemm=True)
            got = _gemm(ub, reg, w_codes, N, 1.0 / sx, 1.0 / swq, cfg)
            assert np.all(got[T:] == gu.CANARY)
            rows = set(rng.integers(0, T, size=16).tolist()) | {0, T - 1}
            for c in range(1, tp):
                rows |= {c * T // tp - 1, c * T // tp}
            rows = np.array(sorted(rows))
            a_codes = of.quantize(x[rows], sx)  # the oracle's own codes
            assert np.array_equal(reg.host()[: T * H].reshape(T, H)[rows], a_codes)
            s = np.float32(np.float32(1.0 / sx) * np.float32(1.0 / swq))
            want = of.ag_rows_fp8(a_codes, w_codes, N, s, 1.0)
            _check_tol(got[rows], want, a_codes, w_codes, 1.0 / sx, 1.0 / swq, f"fp8 qkv T={T}")
    finally:
        reg.close()


# ---- reduce-scatter GEMM on E4M3 operands (bf16 partials and sum) -------------------------
def _rs8(ub, reg, a_codes, w_codes, sa, sw, cfg, ldo=None):
    H = reg.hidden
    ldo = ldo or H
    k = a_codes.shape[1]
    out = gu.canary((reg.capacity + 4, ldo))
    ub.ub_gemm_rs_chunked_fp8(reg.h, _dev8(a_codes), k, k, _dev8(w_codes), w_codes.shape[1],
                              sa, sw, out, ldo, cfg)
    torch.cuda.synchronize()
    return gu.host(out)


def _oracle_rs8(capacity, H, tp, a_codes, w_codes, sa, sw, cfg):
    from oracle import manager as om
    T, k = a_codes.shape
    m = om.UserBufferModel(capacity, H, tp)
    assert m.set_active_shape((T, H)) == om.OK
    out = np.full((capacity, H), om.CANARY, np.uint16)
    st, written = of.rs_chunked_fp8(m, a_codes, k, k, w_codes, w_codes.shape[1], out, H, cfg, sa, sw)
    assert st == om.OK and np.all(written == 1)
    return out[:T], m.ws[: tp * T * H].reshape(tp, T, H)


def _as_bf16(codes, transpose=False):
    """E4M3 values are bf16 values: the same numbers as bf16 patterns (for the bounds)."""
    v = of.decode(codes)
    return ob.encode_rne(v.T.copy() if transpose else v)


@pytest.mark.parametrize("tile", ["256x256", "128x256", "256x192"])
def test_rs_fp8_integer_bit_exact_every_schedule(ub, tile):
    """Small-integer codes, power-of-two scales: partials and sums are exact in fp32, so
    partials, ascending and ring-order outputs equal the oracle bit for bit, for every
    chunking, stream count, the device-side loop and every tile shape; the workspace and
    output tails stay untouched."""
    rng = np.random.default_rng(75)
    cap, H, T, tp = 1024, 512, 600, 8
    K = tp * 128
    a = _int_codes(rng, (T, K))
    w = _int_codes(rng, (H, K))
    sa, sw = 2.0 ** -3, 2.0 ** -5
    reg = gu.Registration(ub, cap, H, tp, pad_rows=8)
    gu.force_tile(ub, reg.h, tile)
    try:
        reg.set_T(T)
        for order in ("ascending", "ring"):
            want, want_ws = _oracle_rs8(cap, H, tp, a, w, sa, sw,
                                        op.OverlapCfg(method="pipeline", num_splits=4, reduce_order=order))
            for method, ns, nms, atomic in [("pipeline", 4, 3, False), ("pipeline", 4, 3, True),
                                            ("ring_exchange", 1, 2, False), ("bulk", 3, 1, True),
                                            ("pipeline", 7, 3, False)]:
                print(f"[rs fp8 int] {tile} {order} {method} {ns} {atomic}", flush=True)
                reg.ws_t.fill_(gu.CANARY)
                got = _rs8(ub, reg, a, w, sa, sw, ub.make_cfg(method, ns, nms, atomic_gemm=atomic,
                                                              reduce_order=order))
                assert np.array_equal(got[:T], want), (order, method, ns, atomic)
                assert np.all(got[T:] == gu.CANARY)
                ws = gu.host(reg.ws_t)
                assert np.array_equal(ws[: tp * T * H].reshape(tp, T, H), want_ws)
                assert np.all(ws[tp * T * H:] == gu.CANARY)
    finally:
        reg.close()


def test_rs_fp8_pipelined_pieces_bit_exact(ub):
    """The device-side FP8 reduce-scatter cut into row pieces (debug rs_pieces, each piece's
    reduction on a worker stream after its slice GEMMs): integer codes equal the oracle bit
    for bit in both reduce orders, workspace included, whatever the piece count; the plan
    record reports the pieces taken (cuts on multiples of 1280 rows)."""
    rng = np.random.default_rng(77)
    cap, H, T, tp = 4096, 256, 3000, 4
    K = tp * 64
    a = _int_codes(rng, (T, K))
    w = _int_codes(rng, (H, K))
    sa, sw = 2.0 ** -4, 2.0 ** -3
    reg = gu.Registration(ub, cap, H, tp, pad_rows=8)
    try:
        reg.set_T(T)
        for order in ("ascending", "ring"):
            want, want_ws = _oracle_rs8(cap, H, tp, a, w, sa, sw,
                                        op.OverlapCfg(method="pipeline", num_splits=4, reduce_order=order))
            for pieces, taken in ((1, 0), (2, 2), (3, 3), (8, 3)):
                print(f"[rs fp8 pieces] {order} {pieces}", flush=True)
                ub.ub_debug_set(reg.h, "rs_pieces", pieces)
                reg.ws_t.fill_(gu.CANARY)
                got = _rs8(ub, reg, a, w, sa, sw, ub.make_cfg("pipeline", 4, 3, atomic_gemm=True,
                                                              reduce_order=order))
                assert np.array_equal(got[:T], want), (order, pieces)
                assert np.all(got[T:] == gu.CANARY)
                ws = gu.host(reg.ws_t)
                assert np.array_equal(ws[: tp * T * H].reshape(tp, T, H), want_ws)
                assert ub.ub_debug_plan(reg.h)["rs_pieces"] == taken, (pieces, ub.ub_debug_plan(reg.h))
        ub.ub_debug_set(reg.h, "rs_pieces", 0)
    finally:
        reg.close()


def test_rs_fp8_random_codes_within_tolerance_and_schedule_identical(ub):
    """Codes over every binade, a scale pair whose fp32 product is not a power of two:
    within the bounds of the oracle, and bit-identical across schedules."""
    rng = np.random.default_rng(76)
    cap, H, T, tp = 512, 264, 296, 4
    K = tp * 192
    a = rng.integers(0, 256, size=(T, K)).astype(np.uint8)
    w = rng.integers(0, 256, size=(H, K)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38
    w[(w & 0x7F) == 0x7F] = 0x38
    sa, sw = 0.37, 0.0021
    reg = gu.Registration(ub, cap, H, tp)
    try:
        reg.set_T(T)
        ref = _rs8(ub, reg, a, w, sa, sw, ub.make_cfg("bulk", 1))[:T]
        want, want_ws = _oracle_rs8(cap, H, tp, a, w, sa, sw, op.OverlapCfg(method="bulk"))
        s = float(np.float32(sa) * np.float32(sw))
        st = gu.check_rs_close(ref, want, _as_bf16(a), _as_bf16(w, True), tp, "rs fp8 random",
                               min_equal=0.9, scale=s, slice_err=[
                                   fp8_slice_err(a[:, j * (K // tp):(j + 1) * (K // tp)],
                                                 w[:, j * (K // tp):(j + 1) * (K // tp)], s)
                                   for j in range(tp)])
        print(f"[rs fp8 random] {st}")
        ws = gu.host(reg.ws_t)[: tp * T * H].reshape(tp, T, H)
        ks = K // tp
        for sl in range(tp):
            _check_tol(ws[sl], want_ws[sl], a[:, sl * ks:(sl + 1) * ks], w[:, sl * ks:(sl + 1) * ks],
                       sa, sw, f"rs fp8 partial {sl}", min_equal=0.9)
        for method in ("ring_exchange", "pipeline", "bulk"):
            for ns in (2, 5):
                for atomic in (False, True):
                    got = _rs8(ub, reg, a, w, sa, sw, ub.make_cfg(method, ns, 3, atomic_gemm=atomic, rank=1))
                    assert np.array_equal(got[:T], ref), (method, ns, atomic)
    finally:
        reg.close()


def test_quantize_e4m3_strided_bit_exact(ub):
    """ub_quantize_e4m3 (no handle): strided source and destination, against the oracle's
    quantization; bytes between rows and after the last row untouched."""
    rng = np.random.default_rng(77)
    rows, cols, lds, ldd = 37, 200, 216, 224
    x = _mixed_bf16(rng, (rows, lds))
    src = gu.dev(x)
    dst = torch.full((rows + 1, ldd), CANARY8, dtype=torch.uint8, device="cuda")
    ub.ub_quantize_e4m3(src, lds, dst, ldd, rows, cols, 3.25)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    assert np.array_equal(got[:rows, :cols], of.quantize(x[:, :cols], np.float32(3.25)))
    assert np.all(got[:rows, cols:] == CANARY8) and np.all(got[rows:] == CANARY8)


def test_rs_fp8_fc2_full_size_sampled(ub):
    """The fc2 workload on E4M3 operands: activations [T, 14336] and the weight transposed
    to [4096, 14336] quantized on the GPU with per-tensor scales 448 / amax, the
    device-side loop at T = 16384 and the pipeline schedule at T = 6144.  Sampled rows
    (every chunk and shard boundary) x sampled output columns (every 256-column tile
    boundary) against the oracle within the bound; the GPU's codes of the sampled rows
    and weight rows against the oracle's quantization (the oracle takes its own codes)."""
    w = wl.fc2()
    ra, rw, _ = w.seeds()
    H, tp, K = w.hidden, w.tp, w.k
    a_all = wl.activations(w, w.capacity, ra)
    wt = wl.weights(w, rw)
    amax_a = float(np.max(np.abs(ob.decode(a_all))))
    amax_w = float(np.max(np.abs(ob.decode(wt))))
    sx, swq = np.float32(448.0 / amax_a), np.float32(448.0 / amax_w)
    wt_nk = np.ascontiguousarray(wt.T)
    a8 = torch.empty((w.capacity, K), dtype=torch.uint8, device="cuda")
    w8 = torch.empty((H, K), dtype=torch.uint8, device="cuda")
    ub.ub_quantize_e4m3(gu.dev(a_all), K, a8, K, w.capacity, K, float(sx))
    ub.ub_quantize_e4m3(gu.dev(wt_nk), K, w8, K, H, K, float(swq))
    torch.cuda.synchronize()
    rng = np.random.default_rng(78)
    cols = set(rng.integers(0, H, size=40).tolist()) | {0, H - 1}
    for b in range(256, H, 256):
        cols |= {b - 1, b}
    cols = np.array(sorted(cols))
    w_codes = of.quantize(wt_nk[cols], swq)  # [len(cols), K]: output columns `cols`
    assert np.array_equal(w8[torch.as_tensor(cols, device="cuda")].cpu().numpy(), w_codes)
    reg = gu.Registration(ub, w.capacity, H, tp, pad_rows=8)
    try:
        for T, atomic in ((w.capacity, True), (6144, False)):
            print(f"[rs fp8 fc2] T={T} atomic={atomic}", flush=True)
            reg.set_T(T)
            out = gu.canary((w.capacity + 8, H))
            cfg = ub.make_cfg(w.method, w.num_splits, w.num_max_streams, atomic_gemm=atomic)
            ub.ub_gemm_rs_chunked_fp8(reg.h, a8, K, K, w8, K, 1.0 / sx, 1.0 / swq, out, H, cfg)
            torch.cuda.synchronize()
            oh = gu.host(out)
            assert np.all(oh[T:] == gu.CANARY)
            rows = set(rng.integers(0, T, size=12).tolist()) | {0, T - 1}
            for c in range(1, w.num_splits):
                rows |= {(c * T) // w.num_splits - 1, (c * T) // w.num_splits}
            for r in range(1, tp):
                rows |= {r * T // tp - 1, r * T // tp}
            rows = np.array(sorted(rows))
            a_codes = of.quantize(a_all[rows], sx)
            assert np.array_equal(a8[torch.as_tensor(rows, device="cuda")].cpu().numpy(), a_codes)
            want, _ = of.rs_rows_fp8(rows, a_codes, w_codes, T, tp, 1.0 / sx, 1.0 / swq)
            s = float(np.float32(1.0 / sx) * np.float32(1.0 / swq))
            st = gu.check_rs_close(oh[rows][:, cols], want, _as_bf16(a_codes), _as_bf16(w_codes, True),
                                   tp, f"rs fp8 fc2 T={T}", min_equal=0.9, scale=s, slice_err=[
                                       fp8_slice_err(a_codes[:, j * (K // tp):(j + 1) * (K // tp)],
                                                     w_codes[:, j * (K // tp):(j + 1) * (K // tp)], s)
                                       for j in range(tp)])
            print(f"[rs fp8 fc2] T={T} {st}", flush=True)
    finally:
        reg.close()


def test_mfma_block_sum_model(ub):
    """The summation model behind the FP8 bounds, measured through ub_gemm_ag_chunked_fp8:
    448*448 + 2**j - 448*448 gives 2**j when the three products sit in three 64-code blocks
    (an fp32 accumulator: j >= -6 survive next to 2**17.6) and, inside one block, 2**j for
    j >= 3 and 0 for j <= 2 (bits below 2**(17 - 14) of the block's largest product are
    dropped); alone, every 2**j is exact."""
    cap, H, N = 256, 192, 8
    a = np.zeros((cap, H), np.uint8)
    w = np.zeros((N, H), np.uint8)
    BIG, NBIG, ONE = 0x7E, 0xFE, 0x38   # 448, -448, 1.0
    w[:, 0], w[:, 1], w[:, 2], w[:, 64], w[:, 128] = BIG, ONE, NBIG, ONE, NBIG
    js = list(range(-9, 9))
    for i, j in enumerate(js):
        code = (j + 7) << 3 if j >= -6 else 1 << (j + 9)
        a[3 * i, 0], a[3 * i, 1], a[3 * i, 2] = BIG, code, BIG          # one block
        a[3 * i + 1, 0], a[3 * i + 1, 64], a[3 * i + 1, 128] = BIG, code, BIG  # three blocks
        a[3 * i + 2, 1] = code                                          # alone
    reg = Fp8Reg(ub, cap, H, 1)
    try:
        ub.ub_set_active_shape(reg.h, (cap, H))
        ub.ub_copy_in(reg.h, _dev8(a), cap, 0)
        got = ob.decode(_gemm(ub, reg, w, N, 1.0, 1.0, ub.make_cfg("bulk", 1))[:cap, 0])
        for i, j in enumerate(js):
            assert got[3 * i] == (2.0 ** j if j >= 3 else 0.0), ("one block", j, got[3 * i])
            assert got[3 * i + 1] == (2.0 ** j if j >= -6 else 0.0), ("three blocks", j)
            assert got[3 * i + 2] == 2.0 ** j, ("alone", j)
    finally:
        reg.close()


@pytest.mark.parametrize("tp,T,cap,K,H,pad_a,pad_w,pad_o,order,method,ns,atomic", [
    (1, 40, 64, 128, 64, 0, 0, 0, "ascending", "bulk", 3, False),        # one slice
    (8, 8, 8, 512, 64, 0, 0, 0, "ring", "ring_exchange", 1, True),       # one row per shard
    (6, 294, 300, 384, 136, 64, 32, 8, "ascending", "pipeline", 4, False),  # strided a, w, out
    (6, 294, 300, 384, 136, 64, 32, 8, "ring", "pipeline", 4, True),
    (4, 512, 512, 256, 256, 16, 0, 0, "ascending", "ring_exchange", 1, True),  # T == capacity
])
def test_rs_fp8_edges(ub, tp, T, cap, K, H, pad_a, pad_w, pad_o, order, method, ns, atomic):
    """Integer codes, power-of-two scales (exact partials and sums): one slice, one row per
    shard, row strides beyond k / hidden on every operand, and T equal to the capacity,
    bit for bit against the oracle; nothing written past T rows or between output rows."""
    rng = np.random.default_rng(79 + tp + T)
    lda, ldw, ldo = K + pad_a, K + pad_w, H + pad_o
    a = np.zeros((T, lda), np.uint8)
    w = np.zeros((H, ldw), np.uint8)
    a[:, :K] = _int_codes(rng, (T, K))
    w[:, :K] = _int_codes(rng, (H, K))
    a[:, K:] = 0x7F  # NaN codes past k: a read of them would poison the result
    w[:, K:] = 0x7F
    sa, sw = 2.0 ** -2, 2.0 ** -4
    print(f"[rs fp8 edge] tp={tp} T={T} {order} {method} atomic={atomic}", flush=True)
    reg = gu.Registration(ub, cap, H, tp, pad_rows=8)
    try:
        reg.set_T(T)
        from oracle import manager as om
        m = om.UserBufferModel(cap, H, tp)
        assert m.set_active_shape((T, H)) == om.OK
        want = np.full((cap, ldo), om.CANARY, np.uint16)
        st, written = of.rs_chunked_fp8(m, a, K, lda, w, ldw, want, ldo,
                                        op.OverlapCfg(method=method, num_splits=ns, reduce_order=order), sa, sw)
        assert st == om.OK and np.all(written == 1)
        out = gu.canary((cap + 4, ldo))
        ub.ub_gemm_rs_chunked_fp8(reg.h, _dev8(a), K, lda, _dev8(w), ldw, sa, sw, out, ldo,
                                  ub.make_cfg(method, ns, 3, atomic_gemm=atomic, reduce_order=order))
        torch.cuda.synchronize()
        got = gu.host(out)
        assert np.array_equal(got[:T, :H], want[:T, :H])
        assert np.all(got[:T, H:] == gu.CANARY) and np.all(got[T:] == gu.CANARY)
        ws = gu.host(reg.ws_t)
        assert np.array_equal(ws[: tp * T * H], m.ws[: tp * T * H])
        assert np.all(ws[tp * T * H:] == gu.CANARY)
    finally:
        reg.close()
