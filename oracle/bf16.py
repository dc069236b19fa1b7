"""bf16 <-> float64 for the oracle (test infrastructure only; see ``oracle/__init__``).

The pages fix the UserBuffer element type as unquantized 2-byte bf16 ([TE#3564],
"Implementation approach in the prototype", last paragraph) but say nothing about how a
wider result is rounded to it.  Reading taken: IEEE-754 round-to-nearest, ties-to-even
(RNE), applied once, directly from the exact (fp64) value -- never through fp32, which
would round twice.

bf16 is the top half of an IEEE binary32: 1 sign bit, 8 exponent bits (bias 127), 7
stored significand bits, so 8 significant bits.  Arrays of bf16 are carried as ``uint16``
bit patterns.
"""

import numpy as np

# bf16 keeps 8 significant bits; binary32's smallest normal exponent is -126.
_SIG_BITS = 8
_EMIN = -126
# Largest finite bf16 is (2 - 2**-7) * 2**127; anything that rounds to 2**128 overflows.
_OVERFLOW = 2.0 ** 128


def decode(bits):
    """uint16 bf16 bit patterns -> float64 values (exact).

    A bf16 pattern placed in the high half of a 32-bit word is the binary32 with the same
    value, and every binary32 is exactly a float64.
    """
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns are quieted, not an error
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def encode_rne(x):
    """float64 values -> uint16 bf16 bit patterns, round to nearest, ties to even.

    For finite nonzero x, let e = floor(log2|x|), clamped below at -126 so that the
    subnormal range keeps the fixed spacing 2**-133.  The bf16 values around x are spaced
    q = 2**(e - 7) apart, so the rounded value is rint(x / q) * q, where x / q is exact (q
    is a power of two) and ``np.rint`` rounds halfway cases to the even integer.  A result
    of magnitude 2**128 or more is +-inf.  Zeros keep their sign; NaN maps to the quiet
    NaN 0x7FC0 with the input's sign.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    ax = np.abs(x)
    finite = np.isfinite(x)
    nonzero = finite & (ax != 0.0)

    # frexp: x = m * 2**E with 0.5 <= |m| < 1, hence floor(log2|x|) = E - 1 (exact).
    _, E = np.frexp(np.where(nonzero, x, 1.0))
    e = np.maximum(E.astype(np.int64) - 1, _EMIN)
    q = np.ldexp(1.0, (e - (_SIG_BITS - 1)).astype(np.int32))
    y = np.where(nonzero, np.rint(np.where(nonzero, x, 0.0) / q) * q, x)

    over = nonzero & (np.abs(y) >= _OVERFLOW)
    y = np.where(over, np.copysign(np.inf, x), y)

    # Every y that is finite here is exactly representable in bf16, hence in binary32, so
    # the float32 cast below is exact and its high half is the bf16 pattern.
    with np.errstate(over="ignore", invalid="ignore"):
        f32 = y.astype(np.float32)
    hi = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out[...] = hi
    nan = np.isnan(x)
    if nan.any():
        sign = np.where(np.signbit(x), 0x8000, 0).astype(np.uint16)
        out[nan] = (np.uint16(0x7FC0) | sign)[nan]
    return out


def ulp(bits):
    """Spacing of bf16 values at each given finite bf16 value (float64): the gap from its
    magnitude to the next larger bf16 magnitude, 2**(max(e, -126) - 7) with
    e = floor(log2|v|) (8 significant bits; the subnormals and zero share the smallest
    normal binade's spacing 2**-133).  At a power of two this is the binade above, the
    larger of the two gaps around the value.  Used for error bounds in the tests."""
    v = np.abs(decode(bits))
    _, E = np.frexp(np.where(v > 0, v, 1.0))
    e = np.where(v > 0, np.maximum(E.astype(np.int64) - 1, _EMIN), _EMIN)
    return np.ldexp(1.0, (e - (_SIG_BITS - 1)).astype(np.int32))
