"""Host-side tests of the C-ABI library (no GPU): exports, the buffer-manager state
machine, plan tables against the oracle's independently written plan, argument errors.

ub_init, ub_set_active_shape, the getters and ub_get_plan make no HIP call, and every
argument check of the GEMM entry points runs before the first one, so all of this runs on
the CPU with placeholder (never dereferenced) device addresses.
"""

import ctypes
import itertools
import os
import re

import pytest

from oracle import manager, plan
from tests.test_oracle_plan_manager import constraint_cases

ub = pytest.importorskip("chunked_tp_overlap_amd.ub", reason="libub.so not built")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 16-byte aligned placeholder device address (never dereferenced)


def header_symbols():
    text = open(os.path.join(ROOT, "include", "ub.h")).read()
    return set(re.findall(r"UB_API\s+[\w\s\*]+?\b(ub_\w+)\s*\(", text))


def test_every_declared_symbol_is_exported():
    syms = header_symbols()
    assert syms == set(ub.EXPORTS)
    lib = ctypes.CDLL(ub.LIB_PATH)
    for s in sorted(syms):
        assert hasattr(lib, s), s


def test_library_binds_to_torchs_hip_runtime():
    maps = open("/proc/self/maps").read()
    hip = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(hip) == 1, hip  # exactly one HIP runtime in the process


def test_status_strings():
    for code, name in ub.STATUS.items():
        assert ub.ub_status_string(code) == name


def _handle(capacity, hidden, tp, ws=True):
    ub_bytes, ws_bytes = ub.ub_required_bytes(capacity, hidden, tp)
    return ub.ub_init(capacity, hidden, tp, ub.UB_DTYPE_BF16, FAKE, ub_bytes,
                      FAKE if ws else None, ws_bytes if ws else 0)


def _ws_bytes(cap, hid, tp):
    """The workspace the header describes: tp partial slots of [cap, hid] bf16, then, from the
    next 256-byte boundary, 4-byte tile counters: UB_MAX_STREAMS ranges of (cap/128 + 1) x
    (hid/128) words, or (cap/128 + 64) x (hid/128) for the device-side loop if larger."""
    parts = tp * cap * hid * 2
    rt, ct = -(-cap // 128), -(-hid // 128)
    words = max(ub.UB_MAX_STREAMS * (rt + 1) * ct, (rt + 64) * ct)
    return -(-parts // 256) * 256 + 4 * words


def test_required_bytes_and_registration_errors():
    assert ub.ub_required_bytes(8192, 4096, 8) == (8192 * 4096 * 2, _ws_bytes(8192, 4096, 8))
    assert ub.ub_required_bytes(8192, 4096, 8)[1] == 8 * 8192 * 4096 * 2 + 4 * 8 * 65 * 32
    assert ub.ub_required_bytes(200, 264, 2)[1] == _ws_bytes(200, 264, 2)
    assert ub.ub_required_bytes(512, 256, 2, ub.UB_DTYPE_FP8_E4M3) == (512 * 256, 0)
    for dt in (ub.UB_DTYPE_FP8_E5M2, ub.UB_DTYPE_FP16, 9):
        with pytest.raises(ub.UBError) as e:
            ub.ub_required_bytes(512, 256, 2, dt)
        assert e.value.name == "UB_ERR_DTYPE"
    with pytest.raises(ub.UBError) as e:  # fp8 rows of 16 bytes
        ub.ub_required_bytes(512, 264, 2, ub.UB_DTYPE_FP8_E4M3)
    assert e.value.name == "UB_ERR_INVALID_ARG"
    with pytest.raises(ub.UBError) as e:
        ub.ub_init(512, 256, 2, ub.UB_DTYPE_FP8_E4M3, FAKE, 512 * 256 - 1)
    assert e.value.name == "UB_ERR_BUFFER_TOO_SMALL"
    with pytest.raises(ub.UBError) as e:  # no reduce-scatter workspace for fp8
        ub.ub_init(512, 256, 2, ub.UB_DTYPE_FP8_E4M3, FAKE, 512 * 256, FAKE, 8 << 20)
    assert e.value.name == "UB_ERR_INVALID_ARG"
    with pytest.raises(ub.UBError) as e:
        ub.ub_required_bytes(510, 256, 4)
    assert e.value.name == "UB_ERR_TP_DIVISIBILITY"
    with pytest.raises(ub.UBError) as e:
        ub.ub_init(512, 256, 2, ub.UB_DTYPE_BF16, FAKE, 512 * 256 * 2 - 2)
    assert e.value.name == "UB_ERR_BUFFER_TOO_SMALL"
    with pytest.raises(ub.UBError) as e:
        ub.ub_init(512, 256, 2, ub.UB_DTYPE_BF16, FAKE, 512 * 256 * 2, FAKE, 100)
    assert e.value.name == "UB_ERR_BUFFER_TOO_SMALL"
    with pytest.raises(ub.UBError) as e:
        ub.ub_init(512, 256, 2, ub.UB_DTYPE_BF16, FAKE + 2, 512 * 256 * 2)
    assert e.value.name == "UB_ERR_INVALID_ARG"
    with pytest.raises(ub.UBError) as e:
        ub.ub_init(512, 252, 2, ub.UB_DTYPE_BF16, FAKE, 512 * 256 * 2)
    assert e.value.name == "UB_ERR_INVALID_ARG"


def test_initial_shapes_are_capacity():
    h = _handle(512, 256, 2)
    try:
        assert ub.ub_get_active_shape(h) == (512, 256)
        assert ub.ub_get_capacity_shape(h) == (512, 256)
    finally:
        ub.ub_destroy(h)


@pytest.mark.parametrize("cap,hid,tp,shape,expected", constraint_cases())
def test_constraint_matrix_matches_oracle(cap, hid, tp, shape, expected):
    h = _handle(cap, hid, tp)
    try:
        first = (max(tp, cap // 2 // tp * tp), hid)
        ub.ub_set_active_shape(h, first)
        st = ub.ub_set_active_shape(h, shape, check=False)
        assert ub.STATUS[st] == ("UB_OK" if expected == manager.OK else "UB_ERR_" + expected)
        if expected == manager.OK:
            assert ub.ub_get_active_shape(h) == (shape[0], hid)
        else:
            assert ub.ub_get_active_shape(h) == first  # state unchanged on error
            assert ub.ub_last_error(h) != ""
        assert ub.ub_get_capacity_shape(h) == (cap, hid)
    finally:
        ub.ub_destroy(h)


def _oracle_cfg(method, ns, nms, agg, rank):
    return plan.OverlapCfg(method=method, num_splits=ns, num_max_streams=nms, aggregate=agg, rank=rank)


def test_plan_tables_match_oracle_exhaustively():
    for tp in (1, 2, 4, 8):
        cap = 96 * tp
        h = _handle(cap, 64, tp)
        try:
            for T in sorted({tp, 8 * tp, 24 * tp, 40 * tp, cap}):
                ub.ub_set_active_shape(h, (T, 64))
                for method, ns, nms, agg, op in itertools.product(
                        plan.METHODS, (1, 2, 3, 5, 8, 16), (1, 2, 3, 8, 12), (False, True), ("ag", "rs")):
                    for rank in sorted({0, 1 % tp, tp - 1}):
                        cfg = ub.make_cfg(method, ns, nms, agg, rank=rank)
                        units, S = ub.ub_get_plan(h, cfg, ub.UB_OP_AG if op == "ag" else ub.UB_OP_RS)
                        ref = plan.build(T, tp, _oracle_cfg(method, ns, nms, agg, rank), op,
                                         stream_limit=ub.UB_MAX_STREAMS)
                        assert units == [(u.pos, u.index, u.row0, u.row1, u.stream) for u in ref], \
                            (T, tp, method, ns, nms, agg, rank, op)
                        assert S == plan.num_streams(_oracle_cfg(method, ns, nms, agg, rank), tp,
                                                     ub.UB_MAX_STREAMS)
        finally:
            ub.ub_destroy(h)


def test_plan_of_the_workloads():
    h = _handle(16384, 4096, 8)
    try:
        ub.ub_set_active_shape(h, (12280, 4096))
        units, S = ub.ub_get_plan(h, ub.make_cfg("pipeline", 4), ub.UB_OP_RS)
        assert [(u[2], u[3]) for u in units] == [(0, 3070), (3070, 6140), (6140, 9210), (9210, 12280)]
        assert S == 3
        ub.ub_set_active_shape(h, (16384, 4096))
        units, S = ub.ub_get_plan(h, ub.make_cfg("ring_exchange", 8, aggregate=True), ub.UB_OP_AG)
        assert [u[3] - u[2] for u in units] == [4096] * 4 and S == 3
    finally:
        ub.ub_destroy(h)


def test_gemm_argument_errors_before_any_hip_call():
    h = _handle(512, 256, 2)
    h_nows = _handle(512, 256, 2, ws=False)
    cfg = ub.make_cfg("ring_exchange", 2)
    try:
        def st(name, *args):
            return ub.STATUS[ub.raw_call(name, *args)]
        cp = ctypes.byref(cfg)
        assert st("ub_gemm_ag_chunked", h, None, 384, 384, FAKE, 384, cp, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_gemm_ag_chunked", h, FAKE + 8, 384, 384, FAKE, 384, cp, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_gemm_ag_chunked", h, FAKE, 380, 384, FAKE, 384, cp, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_gemm_ag_chunked", h, FAKE, 384, 376, FAKE, 384, cp, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_gemm_ag_chunked", h, FAKE, 384, 384, FAKE, 100, cp, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_gemm_ag_chunked", h, FAKE, 384, 384, FAKE, 384, None, None) == "UB_ERR_INVALID_ARG"
        bad = ub.make_cfg("ring_exchange", 2, rank=2)
        assert st("ub_gemm_ag_chunked", h, FAKE, 384, 384, FAKE, 384, ctypes.byref(bad), None) == "UB_ERR_INVALID_ARG"
        bad = ub.make_cfg("pipeline", 0)
        assert st("ub_gemm_ag_chunked", h, FAKE, 384, 384, FAKE, 384, ctypes.byref(bad), None) == "UB_ERR_INVALID_ARG"
        bad = ub.make_cfg("pipeline", 2, num_max_streams=0)
        assert st("ub_gemm_ag_chunked", h, FAKE, 384, 384, FAKE, 384, ctypes.byref(bad), None) == "UB_ERR_INVALID_ARG"
        bad = ub.make_cfg("pipeline", 2)
        bad.method = 7
        assert st("ub_gemm_ag_chunked", h, FAKE, 384, 384, FAKE, 384, ctypes.byref(bad), None) == "UB_ERR_INVALID_ARG"
        # reduce-scatter
        assert st("ub_gemm_rs_chunked", h_nows, FAKE, 256, 256, FAKE, 256, FAKE, 256, cp, None) == "UB_ERR_NOT_INITIALIZED"
        assert st("ub_gemm_rs_chunked", h, FAKE, 255, 256, FAKE, 256, FAKE, 256, cp, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_gemm_rs_chunked", h, FAKE, 36, 40, FAKE, 256, FAKE, 256, cp, None) == "UB_ERR_UNSUPPORTED"
        assert st("ub_gemm_rs_chunked", h, FAKE, 256, 248, FAKE, 256, FAKE, 256, cp, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_gemm_rs_chunked", h, FAKE, 256, 256, FAKE, 256, FAKE, 128, cp, None) == "UB_ERR_INVALID_ARG"
        bad = ub.make_cfg("ring_exchange", 2, reduce_order=2)
        assert st("ub_gemm_rs_chunked", h, FAKE, 256, 256, FAKE, 256, FAKE, 256, ctypes.byref(bad), None) == "UB_ERR_INVALID_ARG"
        bad = ub.make_cfg("ring_exchange", 2)
        bad.fuse_reduce = 2
        assert st("ub_gemm_rs_chunked", h, FAKE, 256, 256, FAKE, 256, FAKE, 256, ctypes.byref(bad), None) == "UB_ERR_INVALID_ARG"
        assert "fuse_reduce" in ub.ub_last_error(h)
        assert st("ub_reduce_partials", h_nows, FAKE, 256, 0, None) == "UB_ERR_NOT_INITIALIZED"
        assert st("ub_reduce_partials", h, FAKE, 256, 2, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_reduce_partials", h, FAKE, 256, -1, None) == "UB_ERR_INVALID_ARG"
        # copy-size checks against the active T, not the capacity
        ub.ub_set_active_shape(h, (256, 256))
        assert st("ub_copy_in", h, FAKE, 129, 128, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_copy_in", h, FAKE, 1, -1, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_copy_in", h, FAKE, 0, 256, None) == "UB_OK"  # empty copy, nothing launched
        # null handle
        assert st("ub_set_active_shape", None, None, 2) == "UB_ERR_NOT_INITIALIZED"
        assert ub.raw_call("ub_destroy", None) == 0
    finally:
        ub.ub_destroy(h)
        ub.ub_destroy(h_nows)


def test_cfg_default_fills_every_field():
    """The defaults of the option list, read back through the ctypes layout (a field
    missing or out of place in either struct shows up here)."""
    cfg = ub.ub_overlap_cfg_default()
    got = {n: getattr(cfg, n) for n, _ in cfg._fields_}
    assert got == {"method": ub.UB_RING_EXCHANGE, "num_splits": 1, "num_max_streams": 3,
                   "aggregate": 0, "atomic_gemm": 0, "rank": 0, "use_ce": 1, "num_sm": 0,
                   "set_sm_margin": 0, "reduce_order": ub.UB_REDUCE_ASCENDING, "fuse_reduce": 0}
    # the library writes exactly sizeof(ub_overlap_cfg_t) bytes: a guard word after the
    # struct stays intact
    class Guarded(ctypes.Structure):
        _fields_ = [("cfg", ub.ub_overlap_cfg_t), ("guard", ctypes.c_uint32)]
    g = Guarded()
    g.guard = 0xDEADBEEF
    ub.raw_call("ub_overlap_cfg_default", ctypes.byref(g.cfg))
    assert g.guard == 0xDEADBEEF and g.cfg.reduce_order == 0 and g.cfg.use_ce == 1


def test_arrival_argument_errors_before_any_hip_call():
    h = _handle(512, 256, 2)
    try:
        def st(name, *args):
            return ub.STATUS[ub.raw_call(name, *args)]
        cfg = ub.make_cfg("ring_exchange", 2)
        cp = ctypes.byref(cfg)
        assert st("ub_gemm_ag_arrival", h, None, 0, FAKE, 384, 384, FAKE, 384, cp, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_gemm_ag_arrival", h, FAKE + 8, 0, FAKE, 384, 384, FAKE, 384, cp, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_gemm_ag_arrival", h, FAKE, 0, FAKE, 380, 384, FAKE, 384, cp, None) == "UB_ERR_INVALID_ARG"
        # the device-side chunk loop gates on SDMA deliveries only: a device source through
        # the copy kernel (use_ce=0) is refused before any HIP call
        atomic_ck = ub.make_cfg("ring_exchange", 2, atomic_gemm=True, use_ce=False)
        assert st("ub_gemm_ag_arrival", h, FAKE, 0, FAKE, 384, 384, FAKE, 384, ctypes.byref(atomic_ck), None) == "UB_ERR_UNSUPPORTED"
        assert "SDMA" in ub.ub_last_error(h)
        many_atomic = ub.make_cfg("pipeline", 65, atomic_gemm=True)
        assert st("ub_gemm_ag_arrival", h, FAKE, 0, FAKE, 384, 384, FAKE, 384, ctypes.byref(many_atomic), None) == "UB_ERR_UNSUPPORTED"
        n = ctypes.c_uint32(7)
        assert st("ub_arrival_timeouts", h, ctypes.byref(n)) == "UB_OK" and n.value == 0  # never gated
        assert st("ub_arrival_timeouts", h, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_arrival_timeouts", None, ctypes.byref(n)) == "UB_ERR_NOT_INITIALIZED"
        many = ub.make_cfg("pipeline", 65)
        assert st("ub_gemm_ag_arrival", h, FAKE, 0, FAKE, 384, 384, FAKE, 384, ctypes.byref(many), None) == "UB_ERR_UNSUPPORTED"
        assert st("ub_deliver_chunks", h, None, 0, cp, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_deliver_chunks", h, FAKE, 0, ctypes.byref(many), None) == "UB_ERR_UNSUPPORTED"
        assert st("ub_deliver_chunks", h, FAKE, 0, None, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_deliver_chunks", None, FAKE, 0, cp, None) == "UB_ERR_NOT_INITIALIZED"
    finally:
        ub.ub_destroy(h)


def test_fp8_handle_argument_errors_before_any_hip_call():
    h = ub.ub_init(512, 256, 2, ub.UB_DTYPE_FP8_E4M3, FAKE, 512 * 256)
    hb = _handle(512, 256, 2)
    try:
        def st(name, *args):
            return ub.STATUS[ub.raw_call(name, *args)]
        cfg = ub.make_cfg("ring_exchange", 2)
        cp = ctypes.byref(cfg)
        f = ctypes.c_float
        # bf16-only entry points refuse an fp8 buffer, and the reverse
        assert st("ub_gemm_ag_chunked", h, FAKE, 384, 384, FAKE, 384, cp, None) == "UB_ERR_DTYPE"
        assert st("ub_gemm_ag_arrival", h, FAKE, 0, FAKE, 384, 384, FAKE, 384, cp, None) == "UB_ERR_DTYPE"
        assert st("ub_deliver_chunks", h, FAKE, 0, cp, None) == "UB_ERR_DTYPE"
        assert st("ub_gemm_rs_chunked", h, FAKE, 256, 256, FAKE, 256, FAKE, 256, cp, None) == "UB_ERR_DTYPE"
        assert st("ub_reduce_partials", h, FAKE, 256, 0, None) == "UB_ERR_DTYPE"
        assert st("ub_quantize_in", hb, FAKE, 1, 0, f(1.0), None) == "UB_ERR_DTYPE"
        assert st("ub_gemm_ag_chunked_fp8", hb, FAKE, 384, 256, f(1), f(1), FAKE, 384, cp, None) == "UB_ERR_DTYPE"
        # quantize: alignment, finite scale, size check against the active T
        ub.ub_set_active_shape(h, (256, 256))
        assert st("ub_quantize_in", h, FAKE + 8, 1, 0, f(1.0), None) == "UB_ERR_INVALID_ARG"
        assert st("ub_quantize_in", h, FAKE, 1, 0, f(float("inf")), None) == "UB_ERR_INVALID_ARG"
        assert st("ub_quantize_in", h, FAKE, 129, 128, f(1.0), None) == "UB_ERR_INVALID_ARG"
        assert st("ub_quantize_in", h, FAKE, 0, 256, f(1.0), None) == "UB_OK"
        # fp8 GEMM: weight row stride >= hidden and a multiple of 16, columns multiple of 8
        assert st("ub_gemm_ag_chunked_fp8", h, FAKE, 384, 240, f(1), f(1), FAKE, 384, cp, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_gemm_ag_chunked_fp8", h, FAKE, 384, 264, f(1), f(1), FAKE, 384, cp, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_gemm_ag_chunked_fp8", h, FAKE, 380, 256, f(1), f(1), FAKE, 384, cp, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_gemm_ag_chunked_fp8", h, FAKE, 384, 256, f(1), f(1), FAKE, 376, cp, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_gemm_ag_chunked_fp8", h, FAKE, 384, 256, f(float("nan")), f(1), FAKE, 384, cp, None) == "UB_ERR_INVALID_ARG"
        assert st("ub_gemm_ag_chunked_fp8", h, FAKE, 384, 256, f(1), f(1), FAKE, 384, None, None) == "UB_ERR_INVALID_ARG"
    finally:
        ub.ub_destroy(h)
        ub.ub_destroy(hb)
    h = ub.ub_init(64, 80, 1, ub.UB_DTYPE_FP8_E4M3, FAKE, 64 * 80)
    try:  # hidden not a multiple of the 64-code k step
        cfg = ub.make_cfg("bulk", 1)
        st = ub.raw_call("ub_gemm_ag_chunked_fp8", h, FAKE, 8, 80, ctypes.c_float(1), ctypes.c_float(1),
                         FAKE, 8, ctypes.byref(cfg), None)
        assert ub.STATUS[st] == "UB_ERR_UNSUPPORTED"
    finally:
        ub.ub_destroy(h)


def test_debug_settings_checked_before_any_hip_call():
    """ub_debug_set validates keys and ranges; a forced tile the kernel does not build is
    rejected by the GEMM call before anything is launched; 0/0 restores the library's
    choice.  Nothing but this entry point changes a handle's launches."""
    h = _handle(512, 256, 2)
    try:
        for key, val in (("nope", 1), ("tile_m", -1), ("tile_group", -2),
                         ("arrival_wait_us", -5), ("arrival_drop_flags", 2)):
            with pytest.raises(ub.UBError) as e:
                ub.ub_debug_set(h, key, val)
            assert e.value.name == "UB_ERR_INVALID_ARG"
        cfg = ub.make_cfg("ring_exchange", 2)
        ub.ub_debug_set(h, "tile_m", 192)
        ub.ub_debug_set(h, "tile_n", 128)
        st = ub.raw_call("ub_gemm_ag_chunked", h, FAKE, 384, 384, FAKE, 384, ctypes.byref(cfg), None)
        assert ub.STATUS[st] == "UB_ERR_INVALID_ARG" and "192x128" in ub.ub_last_error(h)
        st = ub.raw_call("ub_gemm_rs_chunked", h, FAKE, 256, 256, FAKE, 256, FAKE, 256,
                         ctypes.byref(cfg), None)
        assert ub.STATUS[st] == "UB_ERR_INVALID_ARG"
        ub.ub_debug_set(h, "tile_m", 0)
        ub.ub_debug_set(h, "tile_n", 0)
        assert ub.ub_debug_last_plan(h) == (0, 0, -1, 0, 0)  # no launch yet
    finally:
        ub.ub_destroy(h)


def test_kernel_timing_modes_checked_before_any_hip_call():
    """ub_set_kernel_timing takes 0 (off), 1 (an event pair per launch) or 2 (chained);
    anything else is rejected and leaves the mode as it was."""
    h = _handle(512, 256, 2)
    try:
        for mode in (0, 1, 2, 0):
            ub.ub_set_kernel_timing(h, mode)
        for bad in (3, -1, 100):
            with pytest.raises(ub.UBError) as e:
                ub.ub_set_kernel_timing(h, bad)
            assert e.value.name == "UB_ERR_INVALID_ARG" and "chained" in ub.ub_last_error(h)
    finally:
        ub.ub_destroy(h)


def test_atomic_gemm_unit_limit_checked_before_any_hip_call():
    h = _handle(1024, 256, 1)
    try:
        cfg = ub.make_cfg("bulk", 65, atomic_gemm=True)
        st = ub.raw_call("ub_gemm_ag_chunked", h, FAKE, 256, 256, FAKE, 256, ctypes.byref(cfg), None)
        assert ub.STATUS[st] == "UB_ERR_UNSUPPORTED"
        assert "64" in ub.ub_last_error(h)
    finally:
        ub.ub_destroy(h)


def test_rs_fp8_and_quantize_argument_errors_before_any_hip_call():
    """ub_gemm_rs_chunked_fp8 runs on a bf16 handle with a workspace (the partials are
    bf16); its operand checks, and ub_quantize_e4m3's, all come before any HIP call."""
    h8 = ub.ub_init(512, 256, 2, ub.UB_DTYPE_FP8_E4M3, FAKE, 512 * 256)
    hb = _handle(512, 256, 2)
    hn = ub.ub_init(512, 256, 2, ub.UB_DTYPE_BF16, FAKE, 512 * 256 * 2)  # no workspace
    try:
        def st(name, *args):
            return ub.STATUS[ub.raw_call(name, *args)]
        cfg = ub.make_cfg("pipeline", 2)
        cp = ctypes.byref(cfg)
        f = ctypes.c_float
        ok = (FAKE, 512, 512, FAKE, 512, f(1), f(1), FAKE, 256, cp, None)
        assert st("ub_gemm_rs_chunked_fp8", h8, *ok) == "UB_ERR_DTYPE"
        assert st("ub_gemm_rs_chunked_fp8", hn, *ok) == "UB_ERR_NOT_INITIALIZED"
        assert st("ub_gemm_rs_chunked_fp8", None, *ok) == "UB_ERR_NOT_INITIALIZED"
        bad = [
            (FAKE, 511, 512, FAKE, 512, f(1), f(1), FAKE, 256, cp, None),        # k % tp
            (FAKE, 512, 496, FAKE, 512, f(1), f(1), FAKE, 256, cp, None),        # lda < k
            (FAKE, 512, 520, FAKE, 512, f(1), f(1), FAKE, 256, cp, None),        # lda % 16
            (FAKE, 512, 512, FAKE, 504, f(1), f(1), FAKE, 256, cp, None),        # ldw < k
            (FAKE, 512, 512, FAKE, 512, f(float("inf")), f(1), FAKE, 256, cp, None),
            (FAKE, 512, 512, FAKE, 512, f(1), f(1), FAKE, 252, cp, None),        # ldo
            (FAKE + 8, 512, 512, FAKE, 512, f(1), f(1), FAKE, 256, cp, None),    # alignment
            (None, 512, 512, FAKE, 512, f(1), f(1), FAKE, 256, cp, None),
            (FAKE, 512, 512, FAKE, 512, f(1), f(1), FAKE, 256, None, None),      # cfg
        ]
        for args in bad:
            assert st("ub_gemm_rs_chunked_fp8", hb, *args) == "UB_ERR_INVALID_ARG", args
        # k / tp not a multiple of the 64-code step
        assert st("ub_gemm_rs_chunked_fp8", hb, FAKE, 192, 192, FAKE, 192, f(1), f(1), FAKE, 256,
                  cp, None) == "UB_ERR_UNSUPPORTED"
        # the fused reduction exists for bf16 operands only
        fused = ub.make_cfg("pipeline", 2, fuse_reduce=True)
        assert st("ub_gemm_rs_chunked_fp8", hb, *ok[:9], ctypes.byref(fused), None) == "UB_ERR_UNSUPPORTED"
        assert "bf16" in ub.ub_last_error(hb)
        # quantize: alignment, strides, sizes, scale; empty is a no-op
        q = "ub_quantize_e4m3"
        assert st(q, FAKE + 8, 64, FAKE, 64, 4, 64, f(1), None) == "UB_ERR_INVALID_ARG"
        assert st(q, FAKE, 64, FAKE + 4, 64, 4, 64, f(1), None) == "UB_ERR_INVALID_ARG"
        assert st(q, FAKE, 60, FAKE, 64, 4, 60, f(1), None) == "UB_ERR_INVALID_ARG"   # cols % 8
        assert st(q, FAKE, 56, FAKE, 64, 4, 64, f(1), None) == "UB_ERR_INVALID_ARG"   # lds < cols
        assert st(q, FAKE, 64, FAKE, 56, 4, 64, f(1), None) == "UB_ERR_INVALID_ARG"   # ldd < cols
        assert st(q, FAKE, 64, FAKE, 64, -1, 64, f(1), None) == "UB_ERR_INVALID_ARG"
        assert st(q, FAKE, 64, FAKE, 64, 4, 64, f(float("nan")), None) == "UB_ERR_INVALID_ARG"
        assert st(q, None, 64, FAKE, 64, 4, 64, f(1), None) == "UB_ERR_INVALID_ARG"
        assert st(q, FAKE, 64, FAKE, 64, 0, 64, f(1), None) == "UB_OK"
        assert st(q, FAKE, 64, FAKE, 64, 4, 0, f(1), None) == "UB_OK"
    finally:
        ub.ub_destroy(h8)
        ub.ub_destroy(hb)
        ub.ub_destroy(hn)
