"""CPU checks of the comparison helpers' zero-reference rules."""
import numpy as np
import pytest

from tests.parity import GRAD_ZERO_ATOL, assert_grad_close, assert_zero_rows


def test_zero_reference_accepts_rounding_level_only():
    ref = np.zeros((3, 2, 8))
    got = np.zeros_like(ref)
    got[2, 0, :] = 5e-7          # cancellation noise of a row whose one key has weight 1
    assert_grad_close(got, ref, "noise")
    got[2, 0, 3] = 4 * GRAD_ZERO_ATOL   # within the element bound, above rounding level
    with pytest.raises(AssertionError, match="rounding level"):
        assert_grad_close(got, ref, "too large")


def test_zero_rows_must_be_exact():
    got = np.zeros((4, 2, 8))
    got[1, 1, 0] = 1e-9
    rows = np.zeros((4, 2), bool)
    rows[0] = True
    assert_zero_rows(got, rows, "exact")
    rows[1, 1] = True
    with pytest.raises(AssertionError, match="no key reaches"):
        assert_zero_rows(got, rows, "nonzero")
