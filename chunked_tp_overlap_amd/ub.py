"""ctypes binding of ``include/ub.h`` -- argument marshalling only.

Every function here has the name of the C entry point it calls and does nothing but
convert arguments (ints, tuples, torch tensors -> pointers and sizes) and turn a non-OK
status into :class:`UBError`.  All work runs in the HIP library ``lib/libub.so``; there is
no fallback: importing this module fails if the library has not been built.

Pointers may be given as ints or as objects with ``data_ptr()`` (torch tensors); streams
as ints, ``None`` (the null stream) or objects with a ``cuda_stream`` attribute.
"""

import ctypes
import os

import torch  # noqa: F401  -- load torch's HIP runtime first; the library binds to it

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libub.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is not built; run `python -m chunked_tp_overlap_amd.build` "
        "(the HIP library is required: there is no CPU fallback)")
_lib = ctypes.CDLL(_LIB_PATH)
LIB_PATH = _LIB_PATH

# ---- enums ------------------------------------------------------------------------------
STATUS = {
    0: "UB_OK", 1: "UB_ERR_INVALID_ARG", 2: "UB_ERR_NDIM", 3: "UB_ERR_ZERO_DIM",
    4: "UB_ERR_CAPACITY", 5: "UB_ERR_HIDDEN_MISMATCH", 6: "UB_ERR_TP_DIVISIBILITY",
    7: "UB_ERR_DTYPE", 8: "UB_ERR_UNSUPPORTED", 9: "UB_ERR_BUFFER_TOO_SMALL",
    10: "UB_ERR_NOT_INITIALIZED", 11: "UB_ERR_HIP",
}
UB_OK = 0
UB_DTYPE_BF16, UB_DTYPE_FP16, UB_DTYPE_FP8_E4M3, UB_DTYPE_FP8_E5M2 = 0, 1, 2, 3
UB_RING_EXCHANGE, UB_PIPELINE, UB_BULK = 0, 1, 2
UB_OP_AG, UB_OP_RS = 0, 1
UB_MAX_STREAMS = 8
METHODS = {"ring_exchange": UB_RING_EXCHANGE, "pipeline": UB_PIPELINE, "bulk": UB_BULK}
UB_REDUCE_ASCENDING, UB_REDUCE_RING = 0, 1
REDUCE_ORDERS = {"ascending": UB_REDUCE_ASCENDING, "ring": UB_REDUCE_RING}

# Every symbol include/ub.h declares.
EXPORTS = (
    "ub_overlap_cfg_default", "ub_required_bytes", "ub_init", "ub_set_active_shape",
    "ub_get_active_shape", "ub_get_capacity_shape", "ub_get_plan", "ub_copy_in",
    "ub_gemm_ag_chunked", "ub_gemm_ag_arrival", "ub_arrival_timeouts", "ub_deliver_chunks",
    "ub_quantize_in",
    "ub_gemm_ag_chunked_fp8", "ub_gemm_rs_chunked", "ub_gemm_rs_chunked_noalloc",
    "ub_gemm_rs_chunked_fp8",
    "ub_quantize_e4m3", "ub_reduce_partials",
    "ub_set_kernel_timing", "ub_get_kernel_timing", "ub_prepare_streams", "ub_debug_set",
    "ub_debug_last_plan", "ub_register_scratch", "ub_destroy", "ub_status_string", "ub_last_error",
)


class UBError(RuntimeError):
    def __init__(self, status, message=""):
        self.status = status
        self.name = STATUS.get(status, f"UB_ERR_{status}")
        super().__init__(f"{self.name}: {message}" if message else self.name)


# ---- structs ----------------------------------------------------------------------------
class ub_overlap_cfg_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "method", "num_splits", "num_max_streams", "aggregate", "atomic_gemm", "rank",
        "use_ce", "num_sm", "set_sm_margin", "reduce_order", "fuse_reduce")]


class ub_plan_unit_t(ctypes.Structure):
    _fields_ = [("pos", ctypes.c_int32), ("unit", ctypes.c_int32), ("row0", ctypes.c_int64),
                ("row1", ctypes.c_int64), ("stream", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class ub_tile_plan_t(ctypes.Structure):
    _fields_ = [("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32), ("cut_row", ctypes.c_int64),
                ("tail_tile_m", ctypes.c_int32), ("tail_tile_n", ctypes.c_int32),
                ("seg_row", ctypes.c_int64), ("nseg", ctypes.c_int32), ("split", ctypes.c_int32),
                ("seg_tile_m", ctypes.c_int32), ("seg_tile_n", ctypes.c_int32),
                ("dispatches", ctypes.c_int32), ("rs_pieces", ctypes.c_int32)]


UB_SCRATCH_COUNTER_BYTES = 256 * 1024
UB_SCRATCH_MIN_BYTES = UB_SCRATCH_COUNTER_BYTES + 64 * 1024


class ub_kernel_stats_t(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64), ("total_ms", ctypes.c_double),
                ("flops", ctypes.c_double), ("bytes", ctypes.c_double)]


_H = ctypes.c_void_p
_P = ctypes.c_void_p
_I32, _I64, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_CFGP = ctypes.POINTER(ub_overlap_cfg_t)

_sig = {
    "ub_overlap_cfg_default": (None, [_CFGP]),
    "ub_required_bytes": (_I32, [_I64, _I64, _I32, _I32, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]),
    "ub_init": (_I32, [ctypes.POINTER(_H), _I64, _I64, _I32, _I32, _P, _SZ, _P, _SZ]),
    "ub_set_active_shape": (_I32, [_H, ctypes.POINTER(_I64), _I32]),
    "ub_get_active_shape": (_I32, [_H, ctypes.POINTER(_I64)]),
    "ub_get_capacity_shape": (_I32, [_H, ctypes.POINTER(_I64)]),
    "ub_get_plan": (_I32, [_H, _CFGP, _I32, ctypes.POINTER(ub_plan_unit_t), _I32,
                           ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
    "ub_copy_in": (_I32, [_H, _P, _I64, _I64, _P]),
    "ub_gemm_ag_chunked": (_I32, [_H, _P, _I64, _I64, _P, _I64, _CFGP, _P]),
    "ub_gemm_ag_arrival": (_I32, [_H, _P, _I32, _P, _I64, _I64, _P, _I64, _CFGP, _P]),
    "ub_deliver_chunks": (_I32, [_H, _P, _I32, _CFGP, _P]),
    "ub_arrival_timeouts": (_I32, [_H, ctypes.POINTER(ctypes.c_uint32)]),
    "ub_quantize_in": (_I32, [_H, _P, _I64, _I64, ctypes.c_float, _P]),
    "ub_gemm_ag_chunked_fp8": (_I32, [_H, _P, _I64, _I64, ctypes.c_float, ctypes.c_float, _P,
                                      _I64, _CFGP, _P]),
    "ub_gemm_rs_chunked": (_I32, [_H, _P, _I64, _I64, _P, _I64, _P, _I64, _CFGP, _P]),
    "ub_gemm_rs_chunked_noalloc": (_I32, [_H, _P, _I64, _I64, _P, _I64, _P, _I64, _CFGP, _P]),
    "ub_gemm_rs_chunked_fp8": (_I32, [_H, _P, _I64, _I64, _P, _I64, ctypes.c_float, ctypes.c_float,
                                      _P, _I64, _CFGP, _P]),
    "ub_quantize_e4m3": (_I32, [_P, _I64, _P, _I64, _I64, _I64, ctypes.c_float, _P]),
    "ub_reduce_partials": (_I32, [_H, _P, _I64, _I32, _P]),
    "ub_set_kernel_timing": (_I32, [_H, _I32]),
    "ub_get_kernel_timing": (_I32, [_H, ctypes.POINTER(ub_kernel_stats_t),
                                    ctypes.POINTER(ub_kernel_stats_t)]),
    "ub_prepare_streams": (_I32, [_H, _I32, _I32]),
    "ub_debug_set": (_I32, [_H, ctypes.c_char_p, _I64]),
    "ub_debug_last_plan": (_I32, [_H, ctypes.POINTER(ub_tile_plan_t)]),
    "ub_register_scratch": (_I32, [_H, _P, _SZ]),
    "ub_destroy": (_I32, [_H]),
    "ub_status_string": (ctypes.c_char_p, [_I32]),
    "ub_last_error": (ctypes.c_char_p, [_H]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


# ---- marshalling helpers ------------------------------------------------------------------
def _ptr(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def _stream(s):
    if s is None:
        return None
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    return int(s)


def _check(st, h=None):
    if st != UB_OK:
        raise UBError(st, ub_last_error(h) if h else "")


def ub_status_string(status):
    return _lib.ub_status_string(int(status)).decode()


def ub_last_error(h):
    return (_lib.ub_last_error(h) or b"").decode()


def ub_overlap_cfg_default():
    cfg = ub_overlap_cfg_t()
    _lib.ub_overlap_cfg_default(ctypes.byref(cfg))
    return cfg


def _reduce_order(x):
    return REDUCE_ORDERS[x] if isinstance(x, str) else int(x)


def make_cfg(method="ring_exchange", num_splits=1, num_max_streams=3, aggregate=False,
             atomic_gemm=False, rank=0, use_ce=True, num_sm=0, set_sm_margin=False,
             reduce_order="ascending", fuse_reduce=False):
    """A ``ub_overlap_cfg_t`` from keyword options ([TE#1344] option names, plus the
    reduce-scatter summation order "ascending" or "ring" and whether the reduce-scatter
    sum runs inside the slice-GEMM launch)."""
    cfg = ub_overlap_cfg_default()
    cfg.method = METHODS[method] if isinstance(method, str) else int(method)
    cfg.num_splits = int(num_splits)
    cfg.num_max_streams = int(num_max_streams)
    cfg.aggregate = int(bool(aggregate))
    cfg.atomic_gemm = int(bool(atomic_gemm))
    cfg.rank = int(rank)
    cfg.use_ce = int(bool(use_ce))
    cfg.num_sm = int(num_sm)
    cfg.set_sm_margin = int(bool(set_sm_margin))
    cfg.reduce_order = _reduce_order(reduce_order)
    cfg.fuse_reduce = int(bool(fuse_reduce))
    return cfg


def ub_required_bytes(capacity, hidden, tp_size, dtype=UB_DTYPE_BF16):
    a, b = _SZ(), _SZ()
    _check(_lib.ub_required_bytes(capacity, hidden, tp_size, dtype, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def _fits(buf, nbytes, what):
    """A tensor passed with a byte count must hold that many bytes (the library trusts the
    count and addresses up to it)."""
    if hasattr(buf, "numel") and hasattr(buf, "element_size"):
        have = buf.numel() * buf.element_size()
        if int(nbytes) > have:
            raise ValueError(f"{what}: {int(nbytes)} bytes declared, the tensor holds {have}")


def ub_init(capacity, hidden, tp_size, dtype, ub_buf, ub_bytes, rs_ws=None, rs_ws_bytes=0):
    _fits(ub_buf, ub_bytes, "ub_buf")
    if rs_ws is not None:
        _fits(rs_ws, rs_ws_bytes, "rs_ws")
    h = _H()
    _check(_lib.ub_init(ctypes.byref(h), capacity, hidden, tp_size, dtype, _ptr(ub_buf),
                        int(ub_bytes), _ptr(rs_ws), int(rs_ws_bytes)))
    return h


def ub_set_active_shape(h, shape, check=True):
    """Returns the status code; raises UBError on failure when ``check``."""
    arr = (_I64 * max(len(shape), 1))(*[int(d) for d in shape])
    st = _lib.ub_set_active_shape(h, arr, len(shape))
    if check:
        _check(st, h)
    return st


def ub_get_active_shape(h):
    out = (_I64 * 2)()
    _check(_lib.ub_get_active_shape(h, out), h)
    return (out[0], out[1])


def ub_get_capacity_shape(h):
    out = (_I64 * 2)()
    _check(_lib.ub_get_capacity_shape(h, out), h)
    return (out[0], out[1])


def ub_get_plan(h, cfg, op=UB_OP_AG, max_units=4096):
    """Returns (list of (pos, unit, row0, row1, stream), n_streams)."""
    buf = (ub_plan_unit_t * max_units)()
    n, s = _I32(), _I32()
    _check(_lib.ub_get_plan(h, ctypes.byref(cfg), op, buf, max_units, ctypes.byref(n), ctypes.byref(s)), h)
    units = [(u.pos, u.unit, u.row0, u.row1, u.stream) for u in buf[: min(n.value, max_units)]]
    return units, s.value


def ub_copy_in(h, src, rows, row_offset, stream=None):
    _check(_lib.ub_copy_in(h, _ptr(src), rows, row_offset, _stream(stream)), h)


def ub_gemm_ag_chunked(h, w, n_cols, ldw, c, ldc, cfg, stream=None):
    _check(_lib.ub_gemm_ag_chunked(h, _ptr(w), n_cols, ldw, _ptr(c), ldc, ctypes.byref(cfg),
                                   _stream(stream)), h)


def _on_host(src):
    return int(hasattr(src, "is_cuda") and not src.is_cuda)


def ub_gemm_ag_arrival(h, src, w, n_cols, ldw, c, ldc, cfg, stream=None):
    """src: a device tensor, or a pinned host tensor (then delivered over PCIe)."""
    _check(_lib.ub_gemm_ag_arrival(h, _ptr(src), _on_host(src), _ptr(w), n_cols, ldw, _ptr(c),
                                   ldc, ctypes.byref(cfg), _stream(stream)), h)


def ub_deliver_chunks(h, src, cfg, stream=None):
    _check(_lib.ub_deliver_chunks(h, _ptr(src), _on_host(src), ctypes.byref(cfg),
                                  _stream(stream)), h)


def ub_arrival_timeouts(h):
    """Tile waits of the arrival-gated device-side chunk loop that hit the time bound."""
    n = ctypes.c_uint32(0)
    _check(_lib.ub_arrival_timeouts(h, ctypes.byref(n)), h)
    return n.value


def ub_quantize_in(h, src, rows, row_offset, scale, stream=None):
    _check(_lib.ub_quantize_in(h, _ptr(src), rows, row_offset, float(scale), _stream(stream)), h)


def ub_gemm_ag_chunked_fp8(h, w, n_cols, ldw, scale_inv_a, scale_inv_w, c, ldc, cfg, stream=None):
    _check(_lib.ub_gemm_ag_chunked_fp8(h, _ptr(w), n_cols, ldw, float(scale_inv_a),
                                       float(scale_inv_w), _ptr(c), ldc, ctypes.byref(cfg),
                                       _stream(stream)), h)


def ub_gemm_rs_chunked(h, a, k, lda, w, ldw, out, ldo, cfg, stream=None):
    _check(_lib.ub_gemm_rs_chunked(h, _ptr(a), k, lda, _ptr(w), ldw, _ptr(out), ldo,
                                   ctypes.byref(cfg), _stream(stream)), h)


def ub_gemm_rs_chunked_noalloc(h, a, k, lda, w, ldw, out, ldo, cfg, stream=None):
    _check(_lib.ub_gemm_rs_chunked_noalloc(h, _ptr(a), k, lda, _ptr(w), ldw, _ptr(out), ldo,
                                   ctypes.byref(cfg), _stream(stream)), h)


def ub_gemm_rs_chunked_fp8(h, a, k, lda, w, ldw, scale_inv_a, scale_inv_w, out, ldo, cfg,
                           stream=None):
    """a: [T, k] E4M3 codes (row stride lda bytes); w: [hidden, k] E4M3 codes (row stride
    ldw bytes); out: [T, hidden] bf16 (row stride ldo elements)."""
    _check(_lib.ub_gemm_rs_chunked_fp8(h, _ptr(a), k, lda, _ptr(w), ldw, float(scale_inv_a),
                                       float(scale_inv_w), _ptr(out), ldo, ctypes.byref(cfg),
                                       _stream(stream)), h)


def ub_quantize_e4m3(src, lds, dst, ldd, rows, cols, scale, stream=None):
    """dst [rows, cols] E4M3 (row stride ldd bytes) = quantized src (bf16, row stride lds)."""
    _check(_lib.ub_quantize_e4m3(_ptr(src), lds, _ptr(dst), ldd, rows, cols, float(scale),
                                 _stream(stream)))


def ub_reduce_partials(h, out, ldo, reduce_order="ascending", stream=None):
    _check(_lib.ub_reduce_partials(h, _ptr(out), ldo, _reduce_order(reduce_order),
                                   _stream(stream)), h)


def ub_set_kernel_timing(h, enable):
    """enable: False/0 off, True/1 an event pair per launch, 2 chained (one event per launch)."""
    _check(_lib.ub_set_kernel_timing(h, int(enable)), h)


def ub_get_kernel_timing(h):
    """Returns (gemm, reduce) dicts: launches, total_ms, flops, bytes."""
    g, r = ub_kernel_stats_t(), ub_kernel_stats_t()
    _check(_lib.ub_get_kernel_timing(h, ctypes.byref(g), ctypes.byref(r)), h)
    conv = lambda s: {"launches": s.launches, "total_ms": s.total_ms, "flops": s.flops, "bytes": s.bytes}
    return conv(g), conv(r)


def ub_prepare_streams(h, num_max_streams=3, copy_stream=False):
    _check(_lib.ub_prepare_streams(h, int(num_max_streams), int(bool(copy_stream))), h)


def ub_debug_set(h, key, value):
    _check(_lib.ub_debug_set(h, key.encode(), int(value)), h)


def ub_debug_last_plan(h, seg=False):
    """(tile_m, tile_n, cut_row, tail_tile_m, tail_tile_n) of the last GEMM launch group, and
    with seg=True also (seg_row, nseg, split, seg_tile_m, seg_tile_n)."""
    p = ub_tile_plan_t()
    _check(_lib.ub_debug_last_plan(h, ctypes.byref(p)), h)
    base = (p.tile_m, p.tile_n, p.cut_row, p.tail_tile_m, p.tail_tile_n)
    return base + (p.seg_row, p.nseg, p.split, p.seg_tile_m, p.seg_tile_n) if seg else base


def ub_debug_plan(h):
    """Every field of the last call's plan record as a dict."""
    p = ub_tile_plan_t()
    _check(_lib.ub_debug_last_plan(h, ctypes.byref(p)), h)
    return {name: getattr(p, name) for name, _ in ub_tile_plan_t._fields_}


def ub_register_scratch(h, buf, nbytes):
    if buf is not None:
        _fits(buf, nbytes, "scratch")
    _check(_lib.ub_register_scratch(h, _ptr(buf), int(nbytes)), h)


def ub_destroy(h):
    _check(_lib.ub_destroy(h))


def raw_call(name, *args):
    """Call a C entry point with already-marshalled arguments and return its raw status
    (for tests of the error paths)."""
    return getattr(_lib, name)(*args)
