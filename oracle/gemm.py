"""Chunked all-gather (AG) and reduce-scatter (RS) GEMMs over the UserBuffer model.

Test infrastructure only (see ``oracle/__init__``).  Definitions followed:

* [MLM#1240], "Why doesn't the hidden dimension appear in initialize_ub()?": the buffer
  holds the communicated activations ``[S, H]``; the column-parallel layers (QKV to
  3H/TP, MLP fc1 to 2H/TP) expand them locally, and the row-parallel layer (fc2) returns
  to ``[S, H]``, whose reduce-scatter leaves each rank a ``[S/TP, H]`` shard.
* [TE#3564], "Implementation approach in the prototype": every view, offset and count
  comes from the active first dimension T; the active data is a contiguous prefix; the
  reduce-scatter partial chunks live inside the workspace's own allocation.
* [TE#1344], option list: the GEMM is cut into chunks (``oracle.plan``); chunking and the
  stream schedule change which rows a launch covers, never the arithmetic.

Arithmetic (the pages fix none; the plain reading):

* AG: C[t, j] = RNE_bf16( sum_k A[t, k] * W[k, j] ) with A the active UserBuffer rows.
* RS: with Ks = K / tp, partial P_s[t, j] = RNE_bf16( sum_{k in slice s} A[t, k] W[k, j] )
  for s = 0..tp-1, each stored as bf16 in the workspace, then
  out[t, j] = RNE_bf16( sum_s P_s[t, j] ), and shard r = out rows [r T/tp, (r+1) T/tp).
* RS in ring order (option ``reduce_order="ring"``; [TE#1344] "ring_exchange": the
  reduce-scatter moves chunks between neighbours): the partials of shard r's rows travel
  around the ring starting at rank r+1; each rank on the way adds its own bf16 partial
  to the arriving bf16 value in fp32 and rounds the sum to bf16 before passing it on,
  and rank r adds last:  acc = P_{r+1};  acc = RNE_bf16(fp32(acc + P_{r+i})) for
  i = 2 .. tp (indices mod tp).  Reading: the pages give neither the direction nor the
  precision of a hop; this is the plain ring with bf16 on the wire and fp32 adds.

Each product of two bf16 values is exact in fp64 (16 significant bits).  The K-term dot
products use fp64 ``np.matmul`` per chunk: exact for integer-valued inputs whose partial
sums stay below 2**53, otherwise within a few fp64 ulps of the exact sum, which changes
the bf16 result only for values within ~1e-12 (relative) of a rounding midpoint.  The tp
partial sum is computed exactly (``exact_sum``).
"""

from fractions import Fraction

import numpy as np

from . import bf16
from . import manager as M
from . import plan as P


def _check_cfg(cfg):
    if cfg.num_splits < 1 or cfg.num_max_streams < 1:
        return M.INVALID_ARG
    if cfg.method not in P.METHODS:
        return M.INVALID_ARG
    return M.OK


def _dot(a, w):
    """fp64 A @ W of decoded bf16 values.  Adding +0.0 makes an exactly-zero sum +0
    whatever the BLAS accumulator started from (reading: sums start from +0)."""
    return (a @ w) + 0.0


def matmul_f64(a_bits, w_bits):
    """fp64 product of two bf16 matrices given as uint16 patterns."""
    return _dot(bf16.decode(a_bits), bf16.decode(w_bits))


def exact_sum(parts):
    """Exact sum along axis 0 of float64 arrays whose entries are bf16 values.

    An fp64 sum of p terms, each with 8 significant bits, is exact when every term is a
    multiple of the smallest term's quantum and the total stays below 2**53 quanta, i.e.
    when the exponent spread of the nonzero terms is at most 53 - 8 - ceil(log2 p).  The
    elements that satisfy this are summed in fp64; any others are summed with rationals.
    """
    parts = np.asarray(parts, dtype=np.float64)
    p = parts.shape[0]
    s = np.sum(parts, axis=0)
    mag = np.abs(parts)
    nz = mag > 0
    _, E = np.frexp(np.where(nz, mag, 1.0))
    emax = np.max(np.where(nz, E, -10**6), axis=0)
    emin = np.min(np.where(nz, E, 10**6), axis=0)
    spread_ok = (emax - emin) <= 53 - 8 - int(np.ceil(np.log2(max(p, 2))))
    bad = np.argwhere(~spread_ok & np.any(nz, axis=0))
    for idx in map(tuple, bad):
        tot = sum((Fraction(float(parts[(i,) + idx])) for i in range(p)), Fraction(0))
        s[idx] = float(tot)  # correctly rounded to fp64 ...
        if Fraction(s[idx]) != tot:  # ... and never needs to be: bf16 sums stay short
            raise ArithmeticError("partial sum not representable in fp64")
    return s


def ag_chunked(model, w_bits, n_cols, ldw, c_bits, ldc, cfg, stream_limit=None):
    """Column-parallel GEMM over the active UserBuffer prefix, one chunk at a time.

    ``w_bits`` is ``[H, ldw]`` (row-major, first ``n_cols`` columns used); ``c_bits`` is
    ``[rows >= T, ldc]`` and receives rows [0, T).  Returns ``(status, written)`` where
    ``written[t]`` counts how many units wrote row t.
    """
    st = _check_cfg(cfg)
    if st != M.OK:
        return st, None
    T, H = model.active_shape
    W = bf16.decode(np.asarray(w_bits).reshape(H, ldw)[:, :n_cols])
    C = np.asarray(c_bits).reshape(-1, ldc)
    written = np.zeros(T, dtype=np.int64)
    for unit in P.build(T, model.tp, cfg, "ag", stream_limit):
        rows = unit.row1 - unit.row0
        if rows == 0:
            continue
        off = model.row_offset_elems(unit.row0)  # from active T (prefix layout)
        A = bf16.decode(model.ub[off: off + rows * H]).reshape(rows, H)
        C[unit.row0: unit.row1, :n_cols] = bf16.encode_rne(_dot(A, W))
        written[unit.row0: unit.row1] += 1
    return M.OK, written


def rs_chunked(model, a_bits, k, lda, w_bits, ldw, out_bits, ldo, cfg, stream_limit=None):
    """Row-parallel GEMM: tp K-slice bf16 partials into the workspace, then their sum.

    ``a_bits`` is ``[rows >= T, lda]`` (first ``k`` columns used), ``w_bits`` is
    ``[k, ldw]`` (first H columns used), ``out_bits`` is ``[rows >= T, ldo]``.  Partial
    slot s of chunk rows [r0, r1) goes to workspace elements starting at
    ``(s * T + r0) * H``.  Returns ``(status, written)``.
    """
    st = _check_cfg(cfg)
    if st != M.OK:
        return st, None
    if cfg.reduce_order not in P.REDUCE_ORDERS:
        return M.INVALID_ARG, None
    T, H = model.active_shape
    tp = model.tp
    if k <= 0 or k % tp != 0:
        return M.INVALID_ARG, None
    ks = k // tp
    A_all = np.asarray(a_bits).reshape(-1, lda)
    W_all = np.asarray(w_bits).reshape(k, ldw)
    out = np.asarray(out_bits).reshape(-1, ldo)
    written = np.zeros(T, dtype=np.int64)
    for unit in P.build(T, tp, cfg, "rs", stream_limit):
        r0, r1 = unit.row0, unit.row1
        rows = r1 - r0
        if rows == 0:
            continue
        A = bf16.decode(A_all[r0:r1, :k])
        parts = []
        for s in range(tp):
            sl = slice(s * ks, (s + 1) * ks)
            ps = bf16.encode_rne(_dot(A[:, sl], bf16.decode(W_all[sl, :H])))
            o = model.partial_offset_elems(s, r0)
            model.ws[o: o + rows * H] = ps.ravel()
            parts.append(bf16.decode(model.ws[o: o + rows * H]).reshape(rows, H))
        if cfg.reduce_order == "ring":
            out[r0:r1, :H] = ring_sum(parts, r0, T, tp)
        else:
            out[r0:r1, :H] = bf16.encode_rne(exact_sum(parts) + 0.0)
        written[r0:r1] += 1
    return M.OK, written


def ring_hop(acc_bits, part_bits):
    """One ring hop: two bf16 values added in fp32 (IEEE round to nearest even), the sum
    rounded to bf16.  The fp32 sum converts to fp64 exactly, so ``encode_rne`` applies the
    single bf16 rounding of the fp32 value."""
    s32 = (bf16.decode(acc_bits).astype(np.float32) + bf16.decode(part_bits).astype(np.float32))
    return bf16.encode_rne(s32.astype(np.float64))


def ring_sum(parts, row0, T, tp):
    """Ring-order reduce-scatter of the partials ``parts[s]`` (float64 arrays of bf16
    values, rows [row0, row0 + rows) of slice s); returns bf16 bits.  Row t belongs to
    shard r = t // (T / tp), whose sum starts at rank (r + 1) mod tp and ends at r."""
    rows = parts[0].shape[0]
    bits = [bf16.encode_rne(p) for p in parts]  # exact: the partials are bf16 values
    out = np.empty(parts[0].shape, dtype=np.uint16)
    shard_rows = T // tp
    t = row0
    while t < row0 + rows:
        r = t // shard_rows
        t1 = min(row0 + rows, (r + 1) * shard_rows)
        sl = slice(t - row0, t1 - row0)
        acc = bits[(r + 1) % tp][sl]
        for i in range(2, tp + 1):
            acc = ring_hop(acc, bits[(r + i) % tp][sl])
        out[sl] = acc
        t = t1
    return out


def shards(out_bits, T, H, tp, ldo=None):
    """The tp contiguous ``[T/tp, H]`` shards of a reduce-scatter output."""
    ldo = H if ldo is None else ldo
    out = np.asarray(out_bits).reshape(-1, ldo)[:T, :H]
    r = T // tp
    return [out[i * r:(i + 1) * r] for i in range(tp)]


# -- single-shot forms, for sampled checks at full size --------------------------------

def ag_rows(a_rows_bits, w_bits, n_cols=None):
    """AG output rows for the given ``[rows, H]`` input rows (rows are independent)."""
    w = np.asarray(w_bits)
    n_cols = w.shape[1] if n_cols is None else n_cols
    return bf16.encode_rne(matmul_f64(a_rows_bits, w[:, :n_cols]))


def rs_rows_ring(rows, a_rows_bits, w_bits, T, tp, H=None):
    """Ring-order reduce-scatter of the given global rows (each row's own shard decides
    its hop order): returns (out bits, partial bits)."""
    a = np.asarray(a_rows_bits)
    w = np.asarray(w_bits)
    H = w.shape[1] if H is None else H
    ks = a.shape[1] // tp
    parts = [bf16.encode_rne(matmul_f64(a[:, s * ks:(s + 1) * ks], w[s * ks:(s + 1) * ks, :H]))
             for s in range(tp)]
    out = np.empty((len(rows), H), dtype=np.uint16)
    for i, t in enumerate(rows):
        dec = [bf16.decode(p[i:i + 1]) for p in parts]
        out[i] = ring_sum(dec, int(t), T, tp)[0]
    return out, parts


def rs_rows(a_rows_bits, w_bits, tp, H=None):
    """RS output rows and bf16 partials for the given ``[rows, K]`` rows of A."""
    a = np.asarray(a_rows_bits)
    w = np.asarray(w_bits)
    H = w.shape[1] if H is None else H
    k = a.shape[1]
    ks = k // tp
    parts = [bf16.encode_rne(matmul_f64(a[:, s * ks:(s + 1) * ks], w[s * ks:(s + 1) * ks, :H]))
             for s in range(tp)]
    out = bf16.encode_rne(exact_sum([bf16.decode(p) for p in parts]) + 0.0)
    return out, parts

