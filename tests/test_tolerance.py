"""The parity bar itself: BF16 spacing and the one-ulp rounding-flip accounting."""
import numpy as np
import pytest

from tests import gpu_helpers as G


def test_bf16_ulp_values():
    assert np.array_equal(G.bf16_ulp(np.array([1.0, 1.5, 2.0, 130.0, -0.75, 0.0])),
                          [2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 1.0, 2.0 ** -8, 2.0 ** -133])


def _ref(n=100000, seed=0):
    return np.random.default_rng(seed).standard_normal(n) * 40


def test_single_ulp_flip_at_large_value_is_counted_not_failed():
    ref = G.bf16_f64(G.O.f64_to_bf16(_ref(20000)))
    got = ref.copy()
    i = int(np.argmax(np.abs(ref)))
    got[i] += np.sign(ref[i]) * G.bf16_ulp(ref[i : i + 1])[0]
    r = G.assert_close("flip", got, ref)
    assert r["flips"] == 1 and r["over"] == 0


def test_two_ulp_error_or_systematic_error_fails():
    ref = G.bf16_f64(G.O.f64_to_bf16(_ref(20000)))
    got = ref.copy()
    i = int(np.argmax(np.abs(ref)))
    got[i] += 2 * G.bf16_ulp(ref[i : i + 1])[0]
    with pytest.raises(AssertionError):
        G.assert_close("two-ulp", got, ref)
    with pytest.raises(AssertionError):
        G.assert_close("scaled", ref * 1.01, ref)        # 1% systematic error: mean bound
    many = ref + G.bf16_ulp(ref) * (np.abs(ref) > 100)   # flips everywhere large: count bound
    with pytest.raises(AssertionError):
        G.assert_close("many", many, ref)


def test_end_to_end_bar_allows_few_ulps_only():
    ref = G.bf16_f64(G.O.f64_to_bf16(_ref(20000)))
    got = ref.copy()
    i = int(np.argmax(np.abs(ref)))
    got[i] += 2 * G.bf16_ulp(ref[i : i + 1])[0]
    G.assert_close_e2e("two-ulp", got, ref)
    got[i] = ref[i] + 3 * G.bf16_ulp(ref[i : i + 1])[0]
    with pytest.raises(AssertionError):
        G.assert_close_e2e("three-ulp", got, ref)
