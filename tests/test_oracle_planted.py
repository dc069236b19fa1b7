"""Planted mistakes in the oracle's arithmetic must be caught by its pins.

Each case swaps one step of the oracle for a plausible wrong version (a dropped K block, a
wrong rounding mode, a dropped slice in the reduce-scatter sum, a sign error, a transposed
operand, a chunk read one row off) and runs a pin from test_oracle_exact against it: the
pin has to fail.  The mistakes are planted in the oracle, on the CPU; nothing here touches
the HIP path.
"""

import numpy as np
import pytest

from oracle import gemm
from tests import test_oracle_exact as pins


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_pins_pass_unmodified():
    pins.test_integer_inputs_exact_at_larger_shape()
    pins.test_integer_inputs_rs_exact()
    pins.test_closed_form_identity_and_one_hot()
    pins.test_square_integer_gemm_exact()


def test_dropped_k_block_is_caught(monkeypatch):
    monkeypatch.setattr(gemm, "_dot", lambda a, w: (a[:, :-16] @ w[:-16]) + 0.0)
    _fails(pins.test_integer_inputs_exact_at_larger_shape)
    _fails(pins.test_integer_inputs_rs_exact)


def test_truncating_rounding_is_caught(monkeypatch):
    def encode_rtz(x):
        x = np.asarray(x, dtype=np.float64)
        bits = x.astype(np.float32).view(np.uint32)  # RNE to fp32 first: exact here
        return (bits >> 16).astype(np.uint16)          # then drop the low half: toward zero

    monkeypatch.setattr(gemm.bf16, "encode_rne", encode_rtz)
    _fails(pins.test_integer_inputs_exact_at_larger_shape)


def test_dropped_slice_in_reduction_is_caught(monkeypatch):
    real = gemm.exact_sum
    monkeypatch.setattr(gemm, "exact_sum", lambda parts: real(list(parts)[:-1]))
    _fails(pins.test_integer_inputs_rs_exact)


def test_sign_error_is_caught(monkeypatch):
    monkeypatch.setattr(gemm, "_dot", lambda a, w: (a[:, 1:] @ w[1:]) - a[:, :1] @ w[:1] + 0.0)
    _fails(pins.test_integer_inputs_exact_at_larger_shape)


def test_transposed_weight_is_caught(monkeypatch):
    # a square weight read transposed (w.T instead of w) keeps every shape valid
    monkeypatch.setattr(gemm, "_dot", lambda a, w: (a @ (w.T if w.shape[0] == w.shape[1] else w)) + 0.0)
    _fails(pins.test_square_integer_gemm_exact)


def test_shifted_row_offset_is_caught(monkeypatch):
    # a chunk's rows read one row late: C row t gets A row t + 1
    real = gemm.M.UserBufferModel.row_offset_elems
    monkeypatch.setattr(gemm.M.UserBufferModel, "row_offset_elems",
                        lambda self, r: real(self, r) + (self.hidden if r > 0 else 0))
    _fails(pins.test_integer_inputs_exact_at_larger_shape)


def _ulp_pins():
    from tests import test_oracle_bf16 as b
    b.test_ulp_is_gap_to_next_pattern_everywhere()
    b.test_ulp_matches_bit_field_rule()


def test_ulp_pins_pass_unmodified():
    _ulp_pins()


def test_ulp_off_by_one_exponent_is_caught(monkeypatch):
    from oracle import bf16
    real = bf16.ulp
    monkeypatch.setattr(bf16, "ulp", lambda bits: real(bits) * 2.0)
    _fails(_ulp_pins)


def test_ulp_binade_below_at_powers_of_two_is_caught(monkeypatch):
    from oracle import bf16

    def below(bits):  # the spacing below |v|: half as large where |v| is a power of two
        v = np.abs(bf16.decode(bits))
        _, E = np.frexp(np.where(v > 0, v, 1.0))
        m = np.where(v > 0, np.frexp(np.where(v > 0, v, 1.0))[0], 0.75)
        e = np.maximum(E.astype(np.int64) - 1 - (m == 0.5), -126)
        return np.ldexp(1.0, (e - 7).astype(np.int32))

    monkeypatch.setattr(bf16, "ulp", below)
    _fails(_ulp_pins)
