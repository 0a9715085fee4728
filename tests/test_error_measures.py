"""The error measures of the GPU parity tests, on the CPU.

A normwise error over a whole tensor hides a single wrong element of a large
state: the per-head element-wise measure must not.  These cases plant such
errors in synthetic arrays and check which gate catches them.
"""
import numpy as np
import pytest

from tests import gpu_support as gs


def _state(N, dk, dv, seed=0):
    return np.random.default_rng(seed).normal(0.0, 0.02, size=(N, dk, dv))


def test_one_wrong_state_element_passes_the_norm_but_not_the_head_gate():
    ref = _state(512, 64, 64)  # 2M elements
    got = ref.copy()
    got[311, 17, 40] += 0.002  # one element off by a tenth of the typical magnitude
    norm, elem = gs.state_errors(got, ref)
    assert norm <= gs.STATE_GATE          # invisible to the normwise gate
    assert elem > 100 * gs.ELEM_STATE_GATE      # glaring per head
    with pytest.raises(AssertionError):
        gs.assert_state(got, ref)


def test_one_wrong_output_element_is_caught():
    rng = np.random.default_rng(1)
    ref = rng.normal(size=(4, 4096, 128))  # [T, N, dv]
    got = ref.copy()
    got[2, 1000, 5] *= 1.01                # a 1 % error in one element
    norm, elem = gs.out_errors(got, ref)
    assert norm <= gs.OUT_GATE
    assert elem > gs.ELEM_OUT_GATE
    with pytest.raises(AssertionError):
        gs.assert_outputs(got, ref)


def test_rounding_level_errors_pass():
    ref = _state(64, 128, 128, seed=2)
    got = (ref.astype(np.float32)).astype(np.float64)  # fp32 rounding of every element
    norm, elem = gs.state_errors(got, ref)
    assert norm < 1e-7 and elem < 1e-7
    gs.assert_state(got, ref)


def test_nan_fails_every_gate():
    ref = _state(4, 8, 8, seed=3)
    got = ref.copy()
    got[1, 2, 3] = np.nan
    assert np.isnan(gs.head_err(got, ref, 2))
    with pytest.raises(AssertionError):
        gs.assert_state(got, ref)


def test_heads_are_scaled_separately():
    """A head whose values are 1000 times smaller than the others' is judged
    against its own size, not the tensor's."""
    ref = _state(8, 16, 16, seed=4)
    ref[5] *= 1e-3
    got = ref.copy()
    got[5] += 1e-3 * 1e-3 * 0.02  # 1e-3 of that head's own scale
    assert gs.head_err(got, ref, 2) > gs.ELEM_STATE_GATE
    assert gs.rel(got, ref) < gs.STATE_GATE


def test_zero_head_uses_the_absolute_error():
    ref = np.zeros((3, 4, 4))
    got = ref.copy()
    got[1, 0, 0] = 1e-7
    assert gs.head_err(got, ref, 2) == pytest.approx(1e-7)


def test_pair_gate_compares_two_gpu_results():
    rng = np.random.default_rng(5)
    a = rng.normal(size=(6, 3, 64))
    b = a * (1 + 1e-7)
    gs.assert_close_pair(a, b, 1, 1e-5)
    b[3, 1, 7] += 1e-2
    with pytest.raises(AssertionError):
        gs.assert_close_pair(a, b, 1, 1e-5)
