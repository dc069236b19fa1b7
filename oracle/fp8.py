"""FP8 (E4M3) UserBuffers for the oracle (test infrastructure only; see ``oracle/__init__``).

The pages name quantized (FP8) UserBuffers and leave them outside the prototype's initial
scope ([TE#3564], "Implementation approach in the prototype", last paragraph: the
prototype targets unquantized 2-byte buffers).  They give no format or scaling rule, so
the plain reading is taken here:

* element format: OCP 8-bit E4M3 ("FN"): 1 sign bit, 4 exponent bits with bias 7, 3
  stored significand bits; subnormals with spacing 2**-9; largest finite value 448; no
  infinities; S.1111.111 is NaN;
* quantization with a per-tensor scale: q = sat(RNE_e4m3(fp32(x * scale))) -- the product
  is formed in fp32 (IEEE round to nearest even), then rounded to the nearest E4M3 value
  (ties to even), and magnitudes beyond 448 saturate to 448; NaN stays NaN;
* the all-gather GEMM on quantized operands, with the weights stored [N, K] (K
  contiguous) as FP8 GEMMs conventionally take them:
      C[t, j] = RNE_bf16( (sum_k qa[t, k] * qw[j, k]) * sa * sw ),
  sa and sw being the per-tensor dequantization factors (1 / scale of each operand).

* the reduce-scatter GEMM on quantized operands: the slice partials are bf16 as on the
  unquantized path, so only the slice GEMMs change:
      P_s[t, j] = RNE_bf16( (sum_{k in slice s} qa[t, k] * qw[j, k]) * fp32(sa * sw) ),
  then the same sum of the partials (ascending, or ring order with a bf16 rounding per hop).
  The product of the two factors is formed once in fp32 (the reading the library's C
  interface states for both FP8 GEMMs).

FP8 codes are carried as uint8 arrays.  Dots of decoded codes are exact in fp64: every
product is a multiple of 2**-18 below 448**2 < 2**17.61, so a dot over K < 2**17 terms is an
integer number of 2**-18 quanta below 2**53 and no partial sum of any order rounds.
"""

import numpy as np

from . import bf16
from . import manager as M
from . import plan as P
from .gemm import exact_sum, ring_sum

_MAX = 448.0
_EMIN = -6          # smallest normal exponent
_MAN = 3            # stored significand bits
NAN_CODE = 0x7F


def decode(codes):
    """uint8 E4M3 codes -> float64 values (exact); NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32))
    sub = np.ldexp(m / 8.0, _EMIN)
    v = np.where(e == 0, sub, normal)
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return sign * v


def encode(x):
    """float64 values -> uint8 E4M3 codes: round to nearest, ties to even, saturating at
    +-448.  For finite nonzero x with e = max(floor(log2|x|), -6) the neighbouring E4M3
    values are spaced q = 2**(e - 3); x / q is exact and ``np.rint`` rounds halves to
    even.  Zeros keep their sign."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    ax = np.abs(x)
    nz = np.isfinite(x) & (ax != 0.0)
    _, E = np.frexp(np.where(nz, ax, 1.0))
    e = np.maximum(E.astype(np.int64) - 1, _EMIN)
    q = np.ldexp(1.0, (e - _MAN).astype(np.int32))
    y = np.where(nz, np.rint(np.where(nz, ax, 0.0) / q) * q, 0.0)
    y = np.minimum(y, _MAX)
    y = np.where(np.isinf(x), _MAX, y)  # saturating conversion
    # y is now an exact E4M3 magnitude: find its code
    _, E2 = np.frexp(np.where(y > 0, y, 1.0))
    e2 = E2.astype(np.int64) - 1
    normal = y >= 2.0 ** _EMIN
    man_n = np.where(normal, np.rint(np.ldexp(y, (-e2).astype(np.int32)) * 8.0 - 8.0), 0)
    code_n = ((e2 + 7) << 3) + man_n.astype(np.int64)
    code_s = np.rint(np.ldexp(y, 9)).astype(np.int64)  # multiples of 2**-9
    code = np.where(normal, code_n, code_s)
    code = np.where(np.signbit(x), code | 0x80, code)
    out[...] = code.astype(np.uint8)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = NAN_CODE | np.where(np.signbit(x[nan]), 0x80, 0).astype(np.uint8)
    return out


def quantize(x_bf16_bits, scale):
    """bf16 patterns -> E4M3 codes of fp32(x * scale) (see the module docstring)."""
    x = bf16.decode(x_bf16_bits).astype(np.float32)
    y = (x * np.float32(scale)).astype(np.float64)  # IEEE fp32 product, then exact widening
    return encode(y)


def ag_chunked_fp8(model_T, ub_codes, hidden, w_codes, n_cols, sa, sw, units):
    """All-gather GEMM over E4M3 operands, unit by unit: rows [r0, r1) of the UserBuffer's
    active prefix (``ub_codes`` flat, row stride ``hidden``) against ``w_codes`` [n_cols,
    >= hidden] (row j = output column j, K contiguous).  Returns the bf16 bits of the T
    rows and a per-row write count.  ``units`` is the plan (``oracle.plan.build``)."""
    T = model_T
    W = decode(np.asarray(w_codes)[:n_cols, :hidden])
    C = np.zeros((T, n_cols), dtype=np.uint16)
    written = np.zeros(T, dtype=np.int64)
    for u in units:
        if u.row1 == u.row0:
            continue
        A = decode(np.asarray(ub_codes)[u.row0 * hidden: u.row1 * hidden]).reshape(-1, hidden)
        dot = (A @ W.T) + 0.0  # exact: products have 8 significant bits, sums stay short
        C[u.row0:u.row1] = bf16.encode_rne(dot * float(sa) * float(sw))
        written[u.row0:u.row1] += 1
    return C, written


def ag_rows_fp8(a_codes_rows, w_codes, n_cols, sa, sw):
    """All-gather GEMM output for the given rows of the quantized UserBuffer (rows are
    independent): bf16 bits of RNE_bf16(sum_k a[t, k] * w[j, k] * sa * sw)."""
    A = decode(a_codes_rows)
    W = decode(np.asarray(w_codes)[:n_cols, :A.shape[1]])
    return bf16.encode_rne(((A @ W.T) + 0.0) * float(sa) * float(sw))


def _dot8(a_codes, w_codes):
    """Exact dot of decoded E4M3 rows: A [t, K] against W [j, K] (see the module notes)."""
    A, W = decode(a_codes), decode(w_codes)
    assert A.shape[1] < 2 ** 17
    return (A @ W.T) + 0.0


def _scale(sa, sw):
    return float(np.float32(sa) * np.float32(sw))


def rs_chunked_fp8(model, a_codes, k, lda, w_codes, ldw, out_bits, ldo, cfg, sa, sw,
                   stream_limit=None):
    """Row-parallel GEMM over E4M3 operands, unit by unit of the reduce-scatter plan:
    ``a_codes`` [rows >= T, lda] (first k columns used), ``w_codes`` [H, ldw] (row j =
    output column j, first k columns used), ``out_bits`` [rows >= T, ldo] bf16.  Slice s
    (columns [s k/tp, (s+1) k/tp)) of chunk rows [r0, r1) gives the bf16 partial P_s,
    written to workspace elements from (s T + r0) H; then the sum as for the bf16
    reduce-scatter.  Returns ``(status, written)``."""
    if cfg.num_splits < 1 or cfg.num_max_streams < 1 or cfg.method not in P.METHODS:
        return M.INVALID_ARG, None
    if cfg.reduce_order not in P.REDUCE_ORDERS:
        return M.INVALID_ARG, None
    T, H = model.active_shape
    tp = model.tp
    if k <= 0 or k % tp != 0:
        return M.INVALID_ARG, None
    ks = k // tp
    s_ = _scale(sa, sw)
    A_all = np.asarray(a_codes).reshape(-1, lda)
    W_all = np.asarray(w_codes).reshape(-1, ldw)[:H]
    out = np.asarray(out_bits).reshape(-1, ldo)
    written = np.zeros(T, dtype=np.int64)
    for unit in P.build(T, tp, cfg, "rs", stream_limit):
        r0, r1 = unit.row0, unit.row1
        rows = r1 - r0
        if rows == 0:
            continue
        parts = []
        for s in range(tp):
            sl = slice(s * ks, (s + 1) * ks)
            ps = bf16.encode_rne(_dot8(A_all[r0:r1, sl], W_all[:, sl]) * s_)
            o = model.partial_offset_elems(s, r0)
            model.ws[o: o + rows * H] = ps.ravel()
            parts.append(bf16.decode(model.ws[o: o + rows * H]).reshape(rows, H))
        if cfg.reduce_order == "ring":
            out[r0:r1, :H] = ring_sum(parts, r0, T, tp)
        else:
            out[r0:r1, :H] = bf16.encode_rne(exact_sum(parts) + 0.0)
        written[r0:r1] += 1
    return M.OK, written


def rs_rows_fp8(rows, a_codes_rows, w_codes, T, tp, sa, sw, ring=False):
    """Reduce-scatter output for the given global rows (``a_codes_rows`` [len(rows), K]
    E4M3 codes, ``w_codes`` [H, >= K]): returns (out bits, list of the tp partials' bits).
    Rows are independent; with ring order each row's own shard (row // (T / tp)) decides
    its hop order."""
    a = np.asarray(a_codes_rows)
    K = a.shape[1]
    ks = K // tp
    w = np.asarray(w_codes)[:, :K]
    s_ = _scale(sa, sw)
    parts = [bf16.encode_rne(_dot8(a[:, s * ks:(s + 1) * ks], w[:, s * ks:(s + 1) * ks]) * s_)
             for s in range(tp)]
    dec = [bf16.decode(p) for p in parts]
    if not ring:
        return bf16.encode_rne(exact_sum(dec) + 0.0), parts
    out = np.empty(parts[0].shape, dtype=np.uint16)
    for i, t in enumerate(rows):
        out[i] = ring_sum([d[i:i + 1] for d in dec], int(t), T, tp)[0]
    return out, parts
