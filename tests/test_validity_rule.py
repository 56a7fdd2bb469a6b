"""The kept-set validity rule the vertical-slash parity tests apply
(helpers.kept_set_or_legal_swap): exact equality with the oracle's top-k,
except swaps of indices whose fp32 sums lie within one fp32 ulp of the k-th
sum. Checked here on hand-made sums, so that the rule itself is pinned: a
legal swap passes, a swap two ulps away or a wrong count fails."""
import numpy as np
import pytest

import helpers as H


def _sums():
    # ten well-separated sums, and two that sit one fp32 ulp apart around
    # the k-th place (k = 4: kept 0, 1, 2 and the larger of 7 / 8)
    s = np.array([9.0, 8.0, 7.0, 0.5, 0.25, 0.125, 0.0625, 3.0, 0.0, 0.01], dtype=np.float64)
    kth = np.float32(3.0)
    s[8] = np.float64(np.nextafter(kth, np.float32(0)))   # one ulp below the k-th sum
    return s


def test_exact_set_passes():
    s = _sums()
    got = np.array([0, 1, 2, 7])
    assert np.array_equal(H.kept_set_or_legal_swap(got, s, 4, "exact"), got)


def test_swap_within_one_ulp_is_legal_and_returned():
    s = _sums()
    got = np.array([0, 1, 2, 8])                 # 8 in, 7 out: one ulp apart
    assert np.array_equal(H.kept_set_or_legal_swap(got, s, 4, "swap"), got)


def test_swap_two_ulps_away_fails():
    s = _sums()
    s[8] = np.float64(np.nextafter(np.nextafter(np.float32(3.0), np.float32(0)), np.float32(0)))
    with pytest.raises(AssertionError):
        H.kept_set_or_legal_swap(np.array([0, 1, 2, 8]), s, 4, "two ulps")


def test_swap_far_from_the_boundary_fails():
    s = _sums()
    with pytest.raises(AssertionError):
        H.kept_set_or_legal_swap(np.array([0, 1, 7, 8]), s, 4, "far")   # 2 (7.0) dropped


def test_wrong_count_or_order_fails():
    s = _sums()
    with pytest.raises(AssertionError):
        H.kept_set_or_legal_swap(np.array([0, 1, 2]), s, 4, "short")
    with pytest.raises(AssertionError):
        H.kept_set_or_legal_swap(np.array([1, 0, 2, 8]), s, 4, "order")
