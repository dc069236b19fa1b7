"""Pins of the oracle's FP8 (E4M3) path: the format and its rounding, quantization, and
the all-gather GEMM on quantized operands."""

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
