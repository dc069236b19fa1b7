"""Pins of the oracle's GEMM arithmetic: exact brute force, integer inputs, closed forms."""

import numpy as np
import pytest

from chunked_tp_overlap_amd import workloads as wl
from oracle import bf16, gemm, manager, plan
from tests import exact


def _cfg(w, **kw):
    d = dict(method=w.method, num_splits=w.num_splits, num_max_streams=w.num_max_streams,
             aggregate=w.aggregate)
    d.update(kw)
    return plan.OverlapCfg(**d)


def _run_ag(capacity, hidden, tp, T, a_bits, w_bits, cfg):
    m = manager.UserBufferModel(capacity, hidden, tp)
    assert m.set_active_shape((T, hidden)) == manager.OK
    m.fill_active(a_bits)
    n = w_bits.shape[1]
    c = np.full((capacity, n), manager.CANARY, np.uint16)
    st, written = gemm.ag_chunked(m, w_bits, n, n, c, n, cfg)
    assert st == manager.OK
    return c, written, m


def _run_rs(capacity, hidden, tp, T, a_bits, w_bits, cfg):
    m = manager.UserBufferModel(capacity, hidden, tp)
    assert m.set_active_shape((T, hidden)) == manager.OK
    k = a_bits.shape[1]
    out = np.full((capacity, hidden), manager.CANARY, np.uint16)
    a = np.full((capacity, k), manager.CANARY, np.uint16)
    a[:T] = a_bits
    st, written = gemm.rs_chunked(m, a, k, k, w_bits, hidden, out, hidden, cfg)
    assert st == manager.OK
    return out, written, m


@pytest.mark.slow
def test_tiny_ag_equals_integer_brute_force():
    """The tiny AG workload (capacity 512, hidden 256, tp 2, T 256, W [256,384], ring),
    bit for bit against exact integer dot products rounded by integer RNE."""
    w = wl.tiny_ag()
    ra, rw, _ = w.seeds()
    a = wl.activations(w, 256, ra)
    wt = wl.weights(w, rw)
    c, written, _ = _run_ag(w.capacity, w.hidden, w.tp, 256, a, wt, _cfg(w))
    ref = exact.gemm_rne(a, wt)
    assert np.array_equal(c[:256], ref)
    assert np.all(written == 1)


@pytest.mark.slow
def test_tiny_rs_equals_integer_brute_force():
    """The tiny RS workload: K=256 in 2 slices of 128; bf16 partials and the final sum,
    bit for bit against the integer brute force."""
    w = wl.tiny_rs()
    ra, rw, _ = w.seeds()
    a = wl.activations(w, 256, ra)
    wt = wl.weights(w, rw)
    out, written, m = _run_rs(w.capacity, w.hidden, w.tp, 256, a, wt, _cfg(w))
    ref, parts = exact.rs_rne(a, wt, w.tp)
    assert np.array_equal(out[:256], ref)
    T, H = 256, w.hidden
    for s in range(w.tp):
        slot = m.ws[s * T * H:(s + 1) * T * H].reshape(T, H)
        assert np.array_equal(slot, parts[s]), s
    assert np.all(written == 1)


def test_integer_inputs_exact_at_larger_shape():
    """Integer inputs in [-2, 2]: every partial sum is an integer far below 2**53, so the
    oracle's fp64 GEMM is exact; it must equal the exact integer product rounded by the
    independent integer RNE, including the ties it produces (e.g. 257 -> 256)."""
    rng = np.random.default_rng(5)
    T, H, N = 192, 2048, 96
    a = wl.integer_bits(rng, (T, H))
    wt = wl.integer_bits(rng, (H, N))
    c, _, _ = _run_ag(256, H, 8, T, a, wt, plan.OverlapCfg(method="bulk", num_splits=3))
    ref = exact.int_valued_gemm_rne(a, wt)
    assert np.array_equal(c[:T], ref)
    vals = np.abs(bf16.decode(ref))
    assert np.any(vals > 256)  # rounding really happens in this set


def test_square_integer_gemm_exact():
    """A square weight (N = H): a transposed operand keeps every shape valid, so only the
    values can show it.  Integer inputs, exact result."""
    rng = np.random.default_rng(15)
    T, H = 40, 96
    a = wl.integer_bits(rng, (T, H))
    wt = wl.integer_bits(rng, (H, H))
    c, _, _ = _run_ag(64, H, 4, T, a, wt, plan.OverlapCfg(method="ring_exchange"))
    assert np.array_equal(c[:T], exact.int_valued_gemm_rne(a, wt))


def test_integer_inputs_rs_exact():
    rng = np.random.default_rng(6)
    T, H, K, tp = 32, 32, 4096, 4
    a = wl.integer_bits(rng, (T, K))
    wt = wl.integer_bits(rng, (K, H))
    out, _, _ = _run_rs(64, H, tp, T, a, wt, plan.OverlapCfg(method="pipeline", num_splits=3))
    ks = K // tp
    parts = [exact.int_valued_gemm_rne(a[:, s * ks:(s + 1) * ks], wt[s * ks:(s + 1) * ks]) for s in range(tp)]
    P = [exact.ints_of(p) for p in parts]  # exact, scaled by 2**133
    ref = np.array([[exact.rne_int(sum(p[i, j] for p in P), exact.SCALE) for j in range(H)]
                    for i in range(T)], dtype=np.uint16)
    assert np.array_equal(out[:T], ref)
    assert np.any(np.abs(bf16.decode(ref)) > 256)  # the final rounding is exercised


@pytest.mark.parametrize("K", [256, 4096])
def test_closed_form_all_ones(K):
    """A = 1, W = 1: every output equals K exactly (K is exact in bf16)."""
    T, N = 16, 24
    a = wl.const_bits((T, K), 1.0)
    wt = wl.const_bits((K, N), 1.0)
    c, _, _ = _run_ag(32, K, 2, T, a, wt, plan.OverlapCfg(num_splits=2))
    assert np.all(bf16.decode(c[:T]) == K)


def test_closed_form_rs_all_ones():
    """fc2 shape in miniature: K = 14336 in 8 slices of 1792 -> each partial is 1792
    (= 7 * 2**8, exact) and the sum is 14336 (= 7 * 2**11, exact)."""
    T, H, K, tp = 16, 8, 14336, 8
    a = wl.const_bits((T, K), 1.0)
    wt = wl.const_bits((K, H), 1.0)
    out, _, m = _run_rs(32, H, tp, T, a, wt, plan.OverlapCfg(method="pipeline", num_splits=4))
    assert np.all(bf16.decode(out[:T]) == 14336)
    assert np.all(bf16.decode(m.ws[: tp * T * H]) == 1792)


def test_closed_form_identity_and_one_hot():
    """Identity W (N = H) returns A bit for bit; a one-hot row of A returns the matching
    row of W bit for bit.  A transposed or shifted operand breaks both."""
    rng = np.random.default_rng(8)
    T, H = 48, 128
    a = wl.normal_bits(rng, (T, H))
    eye = (np.eye(H, dtype=np.uint16) * 0x3F80).astype(np.uint16)
    c, _, _ = _run_ag(64, H, 4, T, a, eye, plan.OverlapCfg(num_splits=4))
    assert np.array_equal(c[:T], a)
    wt = wl.normal_bits(rng, (H, 40), 0.02)
    idx = rng.integers(0, H, size=T)
    onehot = np.zeros((T, H), np.uint16)
    onehot[np.arange(T), idx] = 0x3F80
    c2, _, _ = _run_ag(64, H, 4, T, onehot, wt, plan.OverlapCfg(method="bulk", num_splits=5))
    assert np.array_equal(c2[:T], wt[idx])


def test_rs_with_tp1_is_plain_gemm():
    """With one slice the reduce-scatter is a single GEMM rounded once."""
    rng = np.random.default_rng(9)
    T, H, K = 32, 64, 256
    a = wl.uniform_bits(rng, (T, K))
    wt = wl.uniform_bits(rng, (K, H))
    out, _, _ = _run_rs(32, H, 1, T, a, wt, plan.OverlapCfg(method="pipeline", num_splits=2))
    assert np.array_equal(out[:T], exact.gemm_rne(a, wt))


def test_zero_result_is_positive_zero():
    """An exactly-zero dot product is +0 (the accumulator starts at +0)."""
    T, H, N = 8, 64, 8
    a = wl.const_bits((T, H), -1.0)
    a[:, :] = 0x8000  # -0.0 everywhere
    wt = wl.const_bits((H, N), 3.0)
    c, _, _ = _run_ag(8, H, 1, T, a, wt, plan.OverlapCfg(method="bulk", num_splits=1))
    assert np.all(c[:T] == 0x0000)


def test_exact_sum_falls_back_to_rationals():
    """exact_sum must stay exact when the terms' exponents are far apart."""
    parts = np.array([[2.0 ** 60], [1.0], [-(2.0 ** 60)]])
    assert gemm.exact_sum(parts)[0] == 1.0
