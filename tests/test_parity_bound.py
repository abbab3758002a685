"""The per-element parity bound of the GPU tests (tests/gpu_util.py), on the
CPU: 1e-2 for fp16/bf16 everywhere except where half an output ulp alone
exceeds it, and there half an ulp plus a small float32 slack, never a whole
ulp."""
import numpy as np
import pytest

from gpu_util import ACC_SLACK, compare, element_bounds


def test_bf16_bound_is_the_bar_below_four():
    want = np.array([0.0, 0.3, 1.99, 2.0, 2.646, 3.999])
    bound, wide = element_bounds(want, "bf16")
    assert not wide.any() and np.all(bound == 1e-2)


def test_bf16_half_ulp_from_four():
    want = np.array([4.0, 5.5, 7.99, 8.0, -12.0])
    bound, wide = element_bounds(want, "bf16")
    assert wide.all()
    half = np.array([2.0 ** -6, 2.0 ** -6, 2.0 ** -6, 2.0 ** -5, 2.0 ** -5])
    assert np.allclose(bound, half + ACC_SLACK * np.abs(want))
    # never a whole ulp
    assert np.all(bound < 2 * half)


def test_f16_half_ulp_from_thirty_two():
    bound, wide = element_bounds(np.array([31.9, 32.0, 40.0]), "f16")
    assert list(wide) == [False, True, True]
    assert bound[0] == 1e-2 and abs(bound[1] - (2.0 ** -6 + 32 * ACC_SLACK)) < 1e-12


def test_binade_edge_gets_the_next_half_ulp():
    """|o| just below 8: float32 slack may carry the result to 8, where half
    an ulp is twice as large."""
    want = np.array([8.0 - 1e-4])
    bound, _ = element_bounds(want, "bf16")
    assert bound[0] >= 2.0 ** -5


def test_compare_rejects_errors_over_the_bar():
    want = np.full((2, 3, 8), 2.646)
    got = want.copy()
    got[0, 0, 0] += 1.014e-2                     # an error the old one-ulp bound let through
    with pytest.raises(AssertionError, match="exceed their bound"):
        compare(got, want, "bf16", label="t")
    got[0, 0, 0] = want[0, 0, 0] + 9.9e-3
    compare(got, want, "bf16", label="t")
