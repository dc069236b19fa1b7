"""Exact integer arithmetic used to pin the oracle.  Written independently of ``oracle/``.

Every finite bf16 value is an integer multiple of 2**-133, so scaling by 2**133 turns
bf16 values into Python integers; sums and products are then exact.  Rounding back to
bf16 is done here with integer operations (round to nearest, ties to even), so a mistake
in the oracle's float-based rounding, in its GEMM indexing, or in its chunk loop shows up
as a mismatch against these functions.
"""

import operator

import numpy as np

SCALE = 133  # bf16 value * 2**133 is an integer


def bf16_bits_to_int(b):
    """One bf16 pattern -> integer value * 2**133 (finite patterns only)."""
    b = int(b)
    sign = -1 if (b >> 15) & 1 else 1
    expf = (b >> 7) & 0xFF
    man = b & 0x7F
    if expf == 0xFF:
        raise ValueError("inf/nan has no integer form")
    if expf == 0:
        mag = man  # subnormal: man * 2**-133
    else:
        mag = (128 + man) << (expf - 1)  # (128+man) * 2**(expf-127-7) * 2**133
    return sign * mag


def spacing_int(b):
    """Gap between the magnitude of finite bf16 pattern b and the next larger bf16
    magnitude, as an integer multiple of 2**-133, from the bit fields: patterns that share
    an exponent field are evenly spaced by one unit of the last stored bit, which is
    2**-133 for the subnormals and for exponent field 1, and doubles with each exponent
    field above that.  Past the largest finite magnitude (exponent field 254) the same
    binade's spacing is returned."""
    b = int(b) & 0x7FFF
    expf = b >> 7
    if expf == 0xFF:
        raise ValueError("inf/nan has no spacing")
    return 1 << max(expf - 1, 0)


def ints_of(bits):
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([bf16_bits_to_int(x) for x in flat], dtype=object).reshape(np.shape(bits))


def rne_int(S, frac_bits):
    """bf16 pattern of the exact value S / 2**frac_bits, round to nearest even."""
    S = int(S)
    if S == 0:
        return 0
    neg = S < 0
    a = -S if neg else S
    e = max(a.bit_length() - 1 - frac_bits, -126)  # floor(log2 value), clamped
    shift = frac_bits + e - 7  # quantum 2**(e-7) in units of 2**-frac_bits
    if shift > 0:
        q, r = divmod(a, 1 << shift)
        half = 1 << (shift - 1)
        if r > half or (r == half and (q & 1)):
            q += 1
    else:
        q = a << (-shift)
    if q >= 256:  # carried into the next binade
        q >>= 1
        e += 1
    if e > 127:
        bits = 0x7F80
    elif q < 128:  # subnormal (only possible at e == -126)
        bits = q
    else:
        bits = ((e + 127) << 7) | (q - 128)
    return bits | (0x8000 if neg else 0)


def gemm_rne(a_bits, w_bits):
    """bf16( exact A @ W ) by brute force over Python integers.  Small inputs only."""
    A = ints_of(a_bits)
    W = ints_of(w_bits)
    m, k = A.shape
    k2, n = W.shape
    assert k == k2
    rows = [list(A[i]) for i in range(m)]
    cols = [list(W[:, j]) for j in range(n)]
    out = np.zeros((m, n), dtype=np.uint16)
    for i in range(m):
        ar = rows[i]
        for j in range(n):
            out[i, j] = rne_int(sum(map(operator.mul, ar, cols[j])), 2 * SCALE)
    return out


def gemm_exact_ints(a_bits, w_bits):
    """Exact A @ W as Python integers scaled by 2**266 (object array)."""
    A = ints_of(a_bits)
    W = ints_of(w_bits)
    m, k = A.shape
    _, n = W.shape
    rows = [list(A[i]) for i in range(m)]
    cols = [list(W[:, j]) for j in range(n)]
    out = np.empty((m, n), dtype=object)
    for i in range(m):
        for j in range(n):
            out[i, j] = sum(map(operator.mul, rows[i], cols[j]))
    return out


def rs_rne(a_bits, w_bits, tp):
    """Brute-force row-parallel result: bf16 partial per K slice, exact sum, one RNE.

    Returns (out bits [m, n], list of tp partial bit arrays)."""
    a = np.asarray(a_bits)
    w = np.asarray(w_bits)
    k = a.shape[1]
    ks = k // tp
    parts = [gemm_rne(a[:, s * ks:(s + 1) * ks], w[s * ks:(s + 1) * ks, :]) for s in range(tp)]
    P = [ints_of(p) for p in parts]
    m, n = parts[0].shape
    out = np.zeros((m, n), dtype=np.uint16)
    for i in range(m):
        for j in range(n):
            out[i, j] = rne_int(sum(p[i, j] for p in P), SCALE)
    return out, parts


def int_valued_gemm_rne(a_bits, w_bits):
    """bf16 of A @ W when A and W hold small integers (exact int64 products and sums)."""
    A = ints_of(a_bits)
    W = ints_of(w_bits)
    # integer-valued bf16 -> scaled ints are v * 2**133; undo the scale exactly
    Ai = np.array([[x >> SCALE if x >= 0 else -((-x) >> SCALE) for x in r] for r in A], dtype=np.int64)
    Wi = np.array([[x >> SCALE if x >= 0 else -((-x) >> SCALE) for x in r] for r in W], dtype=np.int64)
    assert np.all(Ai.astype(object) * (1 << SCALE) == A) and np.all(Wi.astype(object) * (1 << SCALE) == W)
    S = Ai @ Wi
    return np.vectorize(lambda s: rne_int(int(s), 0), otypes=[np.uint16])(S)


def round_scaled(a, frac_bits, sig_bits, emin):
    """The value a / 2**frac_bits rounded to `sig_bits` significant bits (exponent clamped
    below at `emin`), round to nearest even; returned at the same scale.  A value that
    already fits is returned unchanged."""
    a = int(a)
    if a == 0:
        return 0
    neg = a < 0
    m = -a if neg else a
    e = max(m.bit_length() - 1 - frac_bits, emin)
    shift = frac_bits + e - (sig_bits - 1)
    if shift <= 0:
        return a
    q, r = divmod(m, 1 << shift)
    half = 1 << (shift - 1)
    if r > half or (r == half and (q & 1)):
        q += 1
    v = q << shift
    return -v if neg else v


def ring_rne(parts_bits, row0, T, tp):
    """Ring reduce-scatter by brute force over integers: shard r = t // (T / tp) starts at
    rank r+1; each hop rounds the exact sum first to fp32 (24 bits) and then to bf16
    (8 bits).  The sign of an exact zero is not modelled (callers avoid zero sums)."""
    P = [ints_of(p) for p in parts_bits]
    rows, n = P[0].shape
    out = np.zeros((rows, n), dtype=np.uint16)
    for i in range(rows):
        r = (row0 + i) // (T // tp)
        for j in range(n):
            acc = P[(r + 1) % tp][i, j]
            for h in range(2, tp + 1):
                acc = round_scaled(acc + P[(r + h) % tp][i, j], SCALE, 24, -126)
                acc = round_scaled(acc, SCALE, 8, -126)
            out[i, j] = rne_int(acc, SCALE)
    return out


def e4m3_to_int(code):
    """One finite E4M3 code -> integer value * 2**9 (written from the bit fields)."""
    c = int(code)
    sign = -1 if c & 0x80 else 1
    e = (c >> 3) & 0xF
    m = c & 7
    if (c & 0x7F) == 0x7F:
        raise ValueError("NaN has no integer form")
    mag = m if e == 0 else (8 + m) << (e - 1)  # (8+m)/8 * 2**(e-7) * 2**9
    return sign * mag


def fp8_gemm_rne(a_codes, w_codes_nk, sa_log2, sw_log2):
    """bf16( sum_k a[t,k] * w[j,k] * 2**sa_log2 * 2**sw_log2 ) by integer brute force
    (w given [N, K]); power-of-two scales keep everything exact."""
    A = [[e4m3_to_int(x) for x in row] for row in np.asarray(a_codes)]
    W = [[e4m3_to_int(x) for x in row] for row in np.asarray(w_codes_nk)]
    out = np.zeros((len(A), len(W)), dtype=np.uint16)
    frac = 18 - sa_log2 - sw_log2  # value = S / 2**frac
    for i, ar in enumerate(A):
        for j, wr in enumerate(W):
            S = sum(x * y for x, y in zip(ar, wr))
            out[i, j] = rne_int(S << max(0, -frac), max(frac, 0))
    return out
