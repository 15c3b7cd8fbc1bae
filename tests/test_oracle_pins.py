"""The CPU oracle against its pins (closed forms, special cases, invariants)."""
import numpy as np
import pytest

import oracle
from tests import pins


def test_p1a_beta_zero_closed_form():
    assert pins.pin_p1a_beta_zero(oracle.recurrence) <= 1e-13


def test_p1b_erase_off_equals_quadratic_gla():
    assert pins.pin_p1b_erase_off(oracle.recurrence) <= 1e-12


def test_p2_one_hot_key_write():
    """One-hot keys: the written row becomes S + (v - S), which is v up to one
    rounding of the difference (a few ulp of |v| <= 4)."""
    assert pins.pin_p2_unit_key_write(oracle.recurrence, one_hot=True) <= 4e-15


def test_p2_unit_key_write():
    assert pins.pin_p2_unit_key_write(oracle.recurrence, one_hot=False) <= 1e-12


def test_p3_chunked_matches_recurrence():
    assert pins.pin_p3_chunked_vs_recurrence(oracle.recurrence, oracle.chunked) <= 1e-10


def test_p4_chunk_size_invariance():
    assert pins.pin_p4_chunk_size_invariance(oracle.chunked) <= 1e-10


def test_p5_single_step_closed_form():
    assert pins.pin_p5_single_step(oracle.recurrence) <= 1e-14


def test_p6_affine_in_initial_state():
    assert pins.pin_p6_affine_in_state(oracle.recurrence) <= 1e-12


def test_p7_split_and_resume():
    assert pins.pin_p7_split_resume(oracle.recurrence) <= 1e-12


def test_p8_packed_varlen_is_bitwise_independent():
    assert pins.pin_p8_varlen_is_independent(oracle.recurrence) == 0.0


def test_p9_gva_is_bitwise_repeated_mha():
    assert pins.pin_p9_gva_is_repeated_mha(oracle.recurrence) == 0.0


def test_p10_key_value_memory():
    assert pins.pin_p10_key_value_memory(oracle.recurrence) <= 1e-14


def test_chunked_intermediates():
    assert pins.pin_chunk_intermediates(oracle.recurrence, oracle.chunked) <= 1e-12


def test_full_head_dim_chunked_matches_recurrence():
    """dk = dv = 128 and chunk 64 (the library's shape) on a short sequence with a tail."""
    x = pins.rand_case(1, 130, 1, 2, 128, 128, 13)
    a = oracle.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], 128 ** -0.5, h0=x["h0"])
    b = oracle.chunked(x["q"], x["k"], x["v"], x["g"], x["beta"], 128 ** -0.5, h0=x["h0"], chunk=64)
    assert np.max(np.abs(a[0] - b[0])) <= 1e-10 and np.max(np.abs(a[1] - b[1])) <= 1e-10


def test_empty_sequences_keep_initial_state():
    """Zero-length sequences produce no output rows and return the initial state."""
    x = pins.rand_case(1, 4, 1, 1, 4, 3, 14, N=3)
    cu = np.array([0, 0, 4, 4], np.int64)
    o, hT = oracle.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], 1.0, cu_seqlens=cu, h0=x["h0"])
    assert np.array_equal(hT[0], x["h0"][0]) and np.array_equal(hT[2], x["h0"][2])
    o2, h2 = oracle.chunked(x["q"], x["k"], x["v"], x["g"], x["beta"], 1.0, cu_seqlens=cu, h0=x["h0"])
    assert np.array_equal(h2[0], x["h0"][0]) and np.max(np.abs(o2 - o)) <= 1e-12


def test_oracle_rejects_bad_sizes():
    x = pins.rand_case(1, 4, 2, 3, 4, 3, 15)  # Hv % Hq != 0
    with pytest.raises(RuntimeError):
        oracle.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], 1.0)
    y = pins.rand_case(1, 4, 1, 1, 4, 3, 16, N=2)
    with pytest.raises(RuntimeError):  # decreasing cu_seqlens
        oracle.recurrence(y["q"], y["k"], y["v"], y["g"], y["beta"], 1.0, cu_seqlens=np.array([0, 3, 2]))


def test_qg_zero_gate_is_q():
    assert pins.pin_qg_zero_gate(oracle.qg) == 0.0


def test_qg_constant_gate_closed_form():
    assert pins.pin_qg_constant_gate(oracle.qg) <= 1e-14


def test_qg_matches_the_chunked_forms_G():
    assert pins.pin_qg_matches_chunked_G(oracle.qg, oracle.chunked) <= 1e-13
