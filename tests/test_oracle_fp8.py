"""Pins of the oracle's FP8 (E4M3) path: the format and its rounding, quantization, the
all-gather GEMM and the reduce-scatter GEMM on quantized operands."""

import os

import numpy as np
import pytest

from oracle import fp8, plan
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_codes.txt")


def _golden():
    out = []
    with open(GOLDEN) as f:
        for ln in f:
            ln = ln.split("#")[0].strip()
            if ln:
                v, c = (x.strip() for x in ln.split("|"))
                out.append((float(v), int(c, 16)))
    return out


@pytest.mark.parametrize("value,code", _golden())
def test_hand_worked_codes(value, code):
    assert int(fp8.encode(np.array([value]))[0]) == code
    if abs(value) <= 448:
        # the exact values decode back (the rounded ones decode to their code's value)
        assert fp8.encode(fp8.decode(np.array([code], np.uint8)))[0] == code


def test_decode_matches_bit_fields_for_every_code():
    for c in range(256):
        v = fp8.decode(np.array([c], np.uint8))[0]
        if (c & 0x7F) == 0x7F:
            assert np.isnan(v)
        else:
            assert v == exact.e4m3_to_int(c) / 2.0 ** 9, c


def test_round_trip_and_ties_exhaustive():
    """Every finite code round-trips; the midpoint of every pair of neighbouring values
    rounds to the one with an even significand; values just off a midpoint round to the
    nearer neighbour."""
    codes = np.array([c for c in range(0x7F)], np.uint8)  # +0 .. 448
    vals = fp8.decode(codes)
    assert np.array_equal(fp8.encode(vals), codes)
    assert np.array_equal(fp8.encode(-vals[1:]), codes[1:] | 0x80)
    lo, hi = vals[:-1], vals[1:]
    mid = (lo + hi) / 2
    even = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:])
    assert np.array_equal(fp8.encode(mid), even)
    eps = (hi - lo) * 1e-6
    assert np.array_equal(fp8.encode(mid - eps), codes[:-1])
    assert np.array_equal(fp8.encode(mid + eps), codes[1:])


def test_saturation_and_specials():
    assert np.all(fp8.encode(np.array([448.0, 463.99, 464.0, 1e30, np.inf])) == 0x7E)
    assert np.all(fp8.encode(np.array([-448.0, -1e30, -np.inf])) == 0xFE)
    assert fp8.encode(np.array([np.nan]))[0] & 0x7F == 0x7F


def test_quantize_uses_the_fp32_product():
    """x * scale is formed in fp32: with a power-of-two scale the product is exact and
    quantize == encode(x * scale)."""
    from oracle import bf16
    rng = np.random.default_rng(61)
    x = bf16.encode_rne(rng.standard_normal(4000) * 3)
    for scale in (1.0, 8.0, 0.25, 2.0 ** 10):
        assert np.array_equal(fp8.quantize(x, scale), fp8.encode(bf16.decode(x) * scale))
    # a non-power-of-two scale: the fp32 product, then one rounding to E4M3
    s = np.float32(1.3)
    want = fp8.encode((bf16.decode(x).astype(np.float32) * s).astype(np.float64))
    assert np.array_equal(fp8.quantize(x, s), want)


def _random_codes(rng, shape, lo=-6, hi=6):
    """Codes of small integers (exact in E4M3)."""
    return fp8.encode(rng.integers(lo, hi + 1, size=shape).astype(np.float64))


@pytest.mark.parametrize("sa_log2,sw_log2", [(0, 0), (-3, 2), (4, -7)])
def test_gemm_equals_integer_brute_force(sa_log2, sw_log2):
    rng = np.random.default_rng(62 + sa_log2)
    T, H, N = 24, 128, 40
    a = _random_codes(rng, (T, H))
    w = _random_codes(rng, (N, H))
    units = plan.build(T, 8, plan.OverlapCfg(method="ring_exchange"), "ag")
    C, written = fp8.ag_chunked_fp8(T, a.ravel(), H, w, N, 2.0 ** sa_log2, 2.0 ** sw_log2, units)
    assert np.all(written == 1)
    assert np.array_equal(C, exact.fp8_gemm_rne(a, w, sa_log2, sw_log2))


def test_gemm_with_random_fp8_values_square_weight():
    """Any finite codes, a square weight: a transposed W keeps the shapes and is only
    visible in the values."""
    rng = np.random.default_rng(63)
    T, H = 16, 64
    a = rng.integers(0, 0x7F, size=(T, H)).astype(np.uint8) | (rng.integers(0, 2, size=(T, H)) * 0x80).astype(np.uint8)
    w = rng.integers(0, 0x7F, size=(H, H)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38
    w[(w & 0x7F) == 0x7F] = 0x38
    units = plan.build(T, 4, plan.OverlapCfg(method="pipeline", num_splits=3), "ag")
    C, _ = fp8.ag_chunked_fp8(T, a.ravel(), H, w, H, 1.0, 2.0 ** -4, units)
    assert np.array_equal(C, exact.fp8_gemm_rne(a, w, 0, -4))


def test_gemm_schedule_free():
    rng = np.random.default_rng(64)
    T, H, N, tp = 40, 64, 24, 8
    a = _random_codes(rng, (T, H))
    w = _random_codes(rng, (N, H))
    ref, _ = fp8.ag_chunked_fp8(T, a.ravel(), H, w, N, 0.5, 0.125,
                                plan.build(T, tp, plan.OverlapCfg(method="bulk"), "ag"))
    for cfg in (plan.OverlapCfg(method="ring_exchange", rank=3),
                plan.OverlapCfg(method="ring_exchange", aggregate=True),
                plan.OverlapCfg(method="pipeline", num_splits=7)):
        got, written = fp8.ag_chunked_fp8(T, a.ravel(), H, w, N, 0.5, 0.125, plan.build(T, tp, cfg, "ag"))
        assert np.array_equal(got, ref) and np.all(written == 1)


def test_planted_mistakes_are_caught(monkeypatch):
    """A wrong exponent bias and a transposed weight each fail a pin."""
    real = fp8.decode
    monkeypatch.setattr(fp8, "decode", lambda c: real(c) * 2.0)  # bias off by one
    with pytest.raises(AssertionError):
        test_decode_matches_bit_fields_for_every_code()
    monkeypatch.setattr(fp8, "decode", real)
    orig = fp8.ag_chunked_fp8

    def transposed(T, ub, H, w, n, sa, sw, units):
        return orig(T, ub, H, np.ascontiguousarray(np.asarray(w)[:n, :H].T), n, sa, sw, units)

    monkeypatch.setattr(fp8, "ag_chunked_fp8", transposed)
    with pytest.raises(AssertionError):
        test_gemm_with_random_fp8_values_square_weight()


# ---- reduce-scatter GEMM on E4M3 operands ------------------------------------------------
def _fp32_parts(x):
    """An fp32 value as (integer mantissa M, exponent e) with x = M * 2**e exactly."""
    m, e = np.frexp(np.float32(x))
    M = int(np.float64(m) * 2 ** 24)
    return M, int(e) - 24


def _rs_fp8_brute(a, w, tp, sa, sw, ring=False, row0=0, T=None):
    """Brute-force reduce-scatter over integers: per slice the exact dot of decoded codes
    (an integer number of 2**-18), times the fp32 product fp32(sa * sw) = M 2**e exactly,
    rounded once to bf16; then the exact sum (one RNE) or the ring hops."""
    M, e = _fp32_parts(np.float32(sa) * np.float32(sw))
    A = [[exact.e4m3_to_int(x) for x in row] for row in a]
    W = [[exact.e4m3_to_int(x) for x in row] for row in w]
    K = len(A[0])
    ks = K // tp
    parts = []
    for s in range(tp):
        p = np.zeros((len(A), len(W)), dtype=np.uint16)
        for i, ar in enumerate(A):
            for j, wr in enumerate(W):
                S = sum(x * y for x, y in zip(ar[s * ks:(s + 1) * ks], wr[s * ks:(s + 1) * ks]))
                num, frac = S * M, 18 - e  # value = num / 2**frac
                p[i, j] = exact.rne_int(num << max(0, -frac), max(frac, 0))
        parts.append(p)
    if ring:
        return exact.ring_rne(parts, row0, T, tp), parts
    P = [exact.ints_of(p) for p in parts]
    out = np.zeros(parts[0].shape, dtype=np.uint16)
    for i in range(out.shape[0]):
        for j in range(out.shape[1]):
            out[i, j] = exact.rne_int(sum(p[i, j] for p in P), exact.SCALE)
    return out, parts


def _rs_fp8_oracle(a, w, tp, sa, sw, cfg, capacity=None):
    from oracle import manager

    T, K = a.shape
    H = w.shape[0]
    m = manager.UserBufferModel(capacity or T, H, tp)
    assert m.set_active_shape((T, H)) == manager.OK
    out = np.full((capacity or T, H), manager.CANARY, np.uint16)
    st, written = fp8.rs_chunked_fp8(m, a, K, K, w, K, out, H, cfg, sa, sw)
    assert st == manager.OK and np.all(written == 1)
    return out[:T], m.ws[: tp * T * H].reshape(tp, T, H), out[T:]


@pytest.mark.parametrize("sa,sw", [(1.0, 1.0), (2.0 ** -3, 2.0 ** 5), (0.37, 0.0021)])
def test_rs_fp8_equals_integer_brute_force(sa, sw):
    """Partials and ascending sum against integer brute force, including a scale pair
    whose fp32 product is not a power of two (the product is exact as M 2**e)."""
    rng = np.random.default_rng(65)
    T, K, H, tp = 12, 128, 24, 4
    a = _random_codes(rng, (T, K))
    w = _random_codes(rng, (H, K))
    out, ws, tail = _rs_fp8_oracle(a, w, tp, sa, sw, plan.OverlapCfg(method="pipeline", num_splits=3),
                                   capacity=T + 4)
    want, parts = _rs_fp8_brute(a, w, tp, sa, sw)
    for s in range(tp):
        assert np.array_equal(ws[s], parts[s]), s
    assert np.array_equal(out, want)
    from oracle import manager
    assert tail.shape[0] == 4 and np.all(tail == manager.CANARY)


def test_rs_fp8_random_codes_every_binade():
    """Codes over the whole E4M3 range (subnormals to 448, both signs)."""
    rng = np.random.default_rng(66)
    T, K, H, tp = 8, 64, 16, 2
    a = rng.integers(0, 256, size=(T, K)).astype(np.uint8)
    w = rng.integers(0, 256, size=(H, K)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38
    w[(w & 0x7F) == 0x7F] = 0x38
    out, ws, _ = _rs_fp8_oracle(a, w, tp, 1.0, 2.0 ** -6, plan.OverlapCfg(method="bulk"))
    want, parts = _rs_fp8_brute(a, w, tp, 1.0, 2.0 ** -6)
    assert np.array_equal(out, want)
    for s in range(tp):
        assert np.array_equal(ws[s], parts[s])


def test_rs_fp8_ring_order_against_brute_force():
    rng = np.random.default_rng(67)
    T, K, H, tp = 16, 128, 16, 4
    a = rng.integers(1, 7, size=(T, K)) * rng.choice([-1, 1], size=(T, K))
    w = rng.integers(1, 7, size=(H, K)) * rng.choice([-1, 1], size=(H, K))
    a, w = fp8.encode(a.astype(np.float64)), fp8.encode(w.astype(np.float64))
    sa, sw = 0.75, 0.0123
    out, _, _ = _rs_fp8_oracle(a, w, tp, sa, sw, plan.OverlapCfg(method="pipeline", num_splits=2,
                                                                 reduce_order="ring"))
    want, _ = _rs_fp8_brute(a, w, tp, sa, sw, ring=True, row0=0, T=T)
    # the brute force does not model the sign of an exact zero: compare values there
    from oracle import bf16 as ob
    assert np.array_equal(ob.decode(out), ob.decode(want))
    assert np.array_equal(out[want != 0], want[want != 0])
    rows = np.array([0, 3, 5, 11, 15])
    got_rows, _ = fp8.rs_rows_fp8(rows, a[rows], w, T, tp, sa, sw, ring=True)
    assert np.array_equal(got_rows, out[rows])


def test_rs_fp8_reduces_to_the_bf16_reduce_scatter():
    """E4M3 values are bf16 values: with unit scales the FP8 path must equal the bf16
    reduce-scatter oracle on the decoded operands (W transposed to [K, H])."""
    from oracle import bf16 as ob
    from oracle import gemm, manager

    rng = np.random.default_rng(68)
    T, K, H, tp = 24, 256, 32, 8
    a = rng.integers(0, 256, size=(T, K)).astype(np.uint8)
    w = rng.integers(0, 256, size=(H, K)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x30
    w[(w & 0x7F) == 0x7F] = 0x30
    cfg = plan.OverlapCfg(method="pipeline", num_splits=4)
    out8, _, _ = _rs_fp8_oracle(a, w, tp, 1.0, 1.0, cfg)
    a16 = ob.encode_rne(fp8.decode(a))
    w16 = ob.encode_rne(fp8.decode(w).T.copy())
    m = manager.UserBufferModel(T, H, tp)
    assert m.set_active_shape((T, H)) == manager.OK
    out16 = np.zeros((T, H), np.uint16)
    st, _ = gemm.rs_chunked(m, a16, K, K, w16, H, out16, H, cfg)
    assert st == manager.OK
    assert np.array_equal(out8, out16)


def test_rs_fp8_schedule_free_and_rows_helper():
    rng = np.random.default_rng(69)
    T, K, H, tp = 40, 128, 16, 8
    a = _random_codes(rng, (T, K))
    w = _random_codes(rng, (H, K))
    ref, _, _ = _rs_fp8_oracle(a, w, tp, 0.5, 0.3, plan.OverlapCfg(method="bulk"))
    for cfg in (plan.OverlapCfg(method="ring_exchange", rank=5),
                plan.OverlapCfg(method="pipeline", num_splits=7, num_max_streams=2)):
        got, _, _ = _rs_fp8_oracle(a, w, tp, 0.5, 0.3, cfg, capacity=64)
        assert np.array_equal(got, ref)
    rows = np.array([0, 7, 19, 39])
    got_rows, parts = fp8.rs_rows_fp8(rows, a[rows], w, T, tp, 0.5, 0.3)
    assert np.array_equal(got_rows, ref[rows]) and len(parts) == tp


TIE_SA, TIE_SW = 1.0 + 2.0 ** -17, 1.0 + 2.0 ** -8 - 2.0 ** -17


def test_rs_fp8_scale_is_one_fp32_product():
    """sa = 1 + 2**-17 and sw = 1 + 2**-8 - 2**-17 are fp32 values whose exact product,
    1 + 2**-8 + 2**-25 - 2**-34, rounds in fp32 to 1 + 2**-8: a bf16 tie, which goes to the
    even 1.0.  The exact product would round up to 1 + 2**-7.  One product of codes 1.0 x
    1.0 in slice 0 (everything else zero) must therefore give 1.0."""
    assert float(np.float32(TIE_SA)) == TIE_SA and float(np.float32(TIE_SW)) == TIE_SW
    assert float(np.float32(TIE_SA) * np.float32(TIE_SW)) == 1.0 + 2.0 ** -8
    T, K, H, tp = 4, 128, 8, 2
    a = np.zeros((T, K), np.uint8)
    w = np.zeros((H, K), np.uint8)
    a[:, 5] = fp8.encode(np.array([1.0]))[0]
    w[:, 5] = fp8.encode(np.array([1.0]))[0]
    out, ws, _ = _rs_fp8_oracle(a, w, tp, TIE_SA, TIE_SW, plan.OverlapCfg(method="bulk"))
    want, parts = _rs_fp8_brute(a, w, tp, TIE_SA, TIE_SW)
    assert np.all(parts[0] == 0x3F80) and np.all(want == 0x3F80)
    assert np.array_equal(out, want) and np.array_equal(ws[0], parts[0])


def test_rs_fp8_planted_mistakes_are_caught(monkeypatch):
    """A transposed weight, a slice taken from the wrong columns, and the scales applied in
    fp64 instead of one fp32 product each fail a pin."""
    orig = fp8.rs_chunked_fp8

    def transposed(model, a, k, lda, w, ldw, out, ldo, cfg, sa, sw, stream_limit=None):
        wt = np.ascontiguousarray(np.asarray(w).reshape(-1, ldw)[:, :k].reshape(k, -1))
        return orig(model, a, k, lda, wt, wt.shape[1], out, ldo, cfg, sa, sw, stream_limit)

    monkeypatch.setattr(fp8, "rs_chunked_fp8", transposed)
    with pytest.raises(Exception):
        test_rs_fp8_equals_integer_brute_force(1.0, 1.0)
    monkeypatch.setattr(fp8, "rs_chunked_fp8", orig)

    real_dot = fp8._dot8
    monkeypatch.setattr(fp8, "_dot8", lambda a, w: real_dot(np.roll(a, 1, axis=1), w))
    with pytest.raises(AssertionError):
        test_rs_fp8_equals_integer_brute_force(1.0, 1.0)
    monkeypatch.setattr(fp8, "_dot8", real_dot)

    monkeypatch.setattr(fp8, "_scale", lambda sa, sw: float(sa) * float(sw))
    with pytest.raises(AssertionError):
        test_rs_fp8_scale_is_one_fp32_product()
