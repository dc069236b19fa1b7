"""Pins for the oracle's bf16 decode / round-to-nearest-even encode (CPU only)."""

import numpy as np
import pytest
import torch

from oracle import bf16
from tests import exact


def test_decode_known_patterns():
    cases = {
        0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0x3F00: 0.5, 0x4380: 256.0,
        0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126, 0x007F: 127 * 2.0 ** -133,
        0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127, 0x0000: 0.0,
    }
    for b, v in cases.items():
        assert bf16.decode(np.array([b], np.uint16))[0] == v, hex(b)
    assert np.isinf(bf16.decode(np.array([0x7F80], np.uint16))[0])
    assert np.signbit(bf16.decode(np.array([0x8000], np.uint16))[0])


@pytest.mark.parametrize("x, bits", [
    (1.0 + 2.0 ** -8, 0x3F80),                # halfway between 1 and 1+2^-7: even is 1
    (1.0 + 3 * 2.0 ** -8, 0x3F82),            # halfway between odd 0x3F81 and even 0x3F82
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),   # just above the midpoint rounds up
    (1.0 + 2.0 ** -8 - 2.0 ** -40, 0x3F80),   # just below rounds down
    (257.0, 0x4380),                          # 257 is a tie between 256 and 258 -> 256
    (259.0, 0x4382),                          # tie between 258 (odd) and 260 (even) -> 260
    (255.5, 0x4380),                          # tie between 255 (odd) and 256 (even): carry
    (2.0 ** -134, 0x0000),                    # half the smallest subnormal ties to 0
    (3 * 2.0 ** -134, 0x0002),                # tie between 1 and 2 subnormal quanta -> 2
    (2.0 ** -126 - 2.0 ** -134, 0x0080),      # rounds up into the normal range
    ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),   # tie between max finite (odd) and 2^128 -> inf
    ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),   # max finite stays
    (-0.0, 0x8000),
    (0.0, 0x0000),
    (-1.5, 0xBFC0),
    (float("inf"), 0x7F80),
    (float("-inf"), 0xFF80),
    (1e300, 0x7F80),
])
def test_encode_rne_hand_cases(x, bits):
    assert int(bf16.encode_rne(np.array([x]))[0]) == bits


def test_encode_nan():
    assert int(bf16.encode_rne(np.array([np.nan]))[0]) & 0x7FC0 == 0x7FC0


def test_round_trip_all_patterns():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((b >> 7) & 0xFF) != 0xFF
    v = bf16.decode(b[finite])
    assert np.array_equal(bf16.encode_rne(v), b[finite])


def test_encode_matches_torch_on_float32_values():
    """For values exactly representable in binary32, one RNE step from fp64 must agree with
    torch's float32 -> bfloat16 cast (also round to nearest even)."""
    rng = np.random.default_rng(7)
    raw = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = raw.view(np.float32)
    f = f[np.isfinite(f)]
    ours = bf16.encode_rne(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_encode_matches_integer_rne_including_ties():
    """Against the independent integer rounding of tests/exact.py, on random fp64 values
    and on exact midpoints between adjacent bf16 values (where double rounding through
    fp32 would go wrong)."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal(20_000) * np.exp2(rng.integers(-140, 120, size=20_000))
    lo = rng.integers(0, 0x7F7F, size=5_000).astype(np.uint16)
    mids = (bf16.decode(lo) + bf16.decode(lo + 1)) / 2  # exact in fp64
    x = np.concatenate([x, mids, -mids])
    ours = bf16.encode_rne(x)
    for xi, oi in zip(x, ours):
        m, e = np.frexp(xi)  # xi = m * 2**e exactly; m has <= 53 bits
        S = int(np.ldexp(m, 60))
        fb = 60 - int(e)
        if fb < 0:
            S <<= -fb
            fb = 0
        assert exact.rne_int(S, fb) == int(oi), (xi, hex(int(oi)))


def test_fp32_double_rounding_would_differ():
    """Sanity of the pin above: a value just above a bf16 midpoint that rounds to the
    midpoint in fp32 must still round up when rounded once from fp64."""
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert int(bf16.encode_rne(np.array([x]))[0]) == 0x3F81
    via32 = torch.tensor([x], dtype=torch.float64).float().to(torch.bfloat16).view(torch.int16)
    assert int(via32.item()) & 0xFFFF == 0x3F80


# ---- spacing (ulp) ----------------------------------------------------------------------
# The spacing of bf16 values at a value sets the tight error bound of every random-input
# parity test, so it is pinned three ways: hand-worked values, the gap to the next
# pattern over every finite pattern (exact integer arithmetic), and the bit-field rule of
# tests/exact.py.

@pytest.mark.parametrize("bits, spacing", [
    (0x3F80, 2.0 ** -7),    # 1.0: 8 significant bits, so the next value is 1 + 2**-7
    (0xBF80, 2.0 ** -7),    # -1.0: the spacing of the magnitude
    (0x437F, 1.0),          # 255 = 1.9921875 * 2**7: spacing 2**0
    (0x4380, 2.0),          # 256 = 2**8: spacing 2**1 (the binade above, not 1 below)
    (0x3F00, 2.0 ** -8),    # 0.5
    (0x0080, 2.0 ** -133),  # smallest normal 2**-126: spacing 2**-133
    (0x0001, 2.0 ** -133),  # smallest subnormal: the fixed subnormal spacing
    (0x007F, 2.0 ** -133),  # largest subnormal
    (0x7F7F, 2.0 ** 120),   # largest finite, (2 - 2**-7) * 2**127
    (0x0000, 2.0 ** -133),  # +0
    (0x8000, 2.0 ** -133),  # -0
])
def test_ulp_hand_cases(bits, spacing):
    assert bf16.ulp(np.array([bits], np.uint16))[0] == spacing


def test_ulp_is_gap_to_next_pattern_everywhere():
    """For every finite non-negative pattern below the largest, the spacing equals the
    exact difference to the next pattern up (integers scaled by 2**133); negative patterns
    take their magnitude's.  The largest finite pattern follows the bit-field rule."""
    b = np.arange(0x7F7F, dtype=np.uint16)           # 0x0000 .. 0x7F7E
    got = bf16.ulp(b)
    gaps = np.array([exact.bf16_bits_to_int(x + 1) - exact.bf16_bits_to_int(x) for x in range(0x7F7F)],
                    dtype=object)
    assert np.array_equal(np.array([int(np.ldexp(v, 133)) for v in got], dtype=object), gaps)
    neg = bf16.ulp(b | np.uint16(0x8000))
    assert np.array_equal(neg, got)


def test_ulp_matches_bit_field_rule():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = b[((b >> 7) & 0xFF) != 0xFF]
    got = bf16.ulp(finite)
    want = np.array([2.0 ** -133 * exact.spacing_int(x) for x in finite])
    assert np.array_equal(got, want)
