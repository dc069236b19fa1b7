"""GPU parity of the FP8 (E4M3) UserBuffer path: ub_quantize_in and ub_gemm_ag_chunked_fp8
against the oracle (oracle.fp8)."""

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


@pytest.mark.parametrize("tile", ["256x256", "128x256"])
def test_gemm_integer_bit_exact_every_schedule(ub, tile, monkeypatch):
    """Small-integer codes, power-of-two scales: every partial sum is exact in fp32, so
    GPU == oracle bit for bit, for every chunking, stream count, rank, aggregate setting,
    the device-side loop, and both tile shapes."""
    monkeypatch.setenv("UBX_GEMM_TILE", tile)
    rng = np.random.default_rng(72)
    cap, H, N, T, tp = 1024, 512, 264, 600, 8
    a = _int_codes(rng, (T, H))
    w = _int_codes(rng, (N, H))
    sa, sw = 2.0 ** -3, 2.0 ** -5
    reg = Fp8Reg(ub, cap, H, tp)
    try:
        ub.ub_set_active_shape(reg.h, (T, H))
        ub.ub_copy_in(reg.h, _dev8(a), T, 0)
        units = op.build(T, tp, op.OverlapCfg(method="bulk"), "ag")
        want, _ = of.ag_chunked_fp8(T, a.ravel(), H, w, N, sa, sw, units)
        for method, ns, nms, agg, rank, atomic in [("ring_exchange", 1, 3, False, 0, False),
                                                  ("ring_exchange", 1, 3, False, 5, True),
                                                  ("ring_exchange", 1, 2, True, 3, True),
                                                  ("pipeline", 7, 3, False, 0, False),
                                                  ("bulk", 3, 1, True, 0, True)]:
            cfg = ub.make_cfg(method, ns, nms, agg, atomic, rank=rank)
            got = _gemm(ub, reg, w, N, sa, sw, cfg)
            assert np.array_equal(got[:T], want), (tile, method, ns, nms, agg, rank, atomic)
            assert np.all(got[T:] == gu.CANARY)
        assert np.all(reg.host()[T * H:] == CANARY8)  # the UB tail was only a canary
    finally:
        reg.close()


def _check_tol(got, want, a_codes, w_codes, sa, sw, what, min_equal=0.98):
    A = of.decode(a_codes)
    W = of.decode(w_codes)
    g = ob.decode(got)
    o = ob.decode(want)
    absdot = (np.abs(A) @ np.abs(W).T) * sa * sw
    K = A.shape[1]
    tight = np.maximum(ob.ulp(got), ob.ulp(want)) + (K + 2) * 2.0 ** -24 * absdot
    gate = 4e-3 * np.outer(np.linalg.norm(A, axis=1), np.linalg.norm(W, axis=1)) * sa * sw
    err = np.abs(g - o)
    assert np.all(err <= gate), f"{what}: gate"
    assert np.all(err <= tight), f"{what}: tight bound"
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
            a_codes = reg.host()[: T * H].reshape(T, H)[rows]
            assert np.array_equal(a_codes, of.quantize(x[rows], sx))
            s = np.float32(np.float32(1.0 / sx) * np.float32(1.0 / swq))
            want = of.ag_rows_fp8(a_codes, w_codes, N, s, 1.0)
            _check_tol(got[rows], want, a_codes, w_codes, 1.0 / sx, 1.0 / swq, f"fp8 qkv T={T}")
    finally:
        reg.close()
