"""Pins of the acceptance gates: known relative errors and planted mistakes."""
import numpy as np
import pytest

from oracle import codecs, tolerance


def _ref():
    return np.random.default_rng(21).standard_normal((64, 256)) * 3


def test_exact_and_small_relative_error_pass():
    r = _ref()
    tolerance.check_e1_e2(r, r)
    st = tolerance.check_e1_e2(r * (1 + 4e-4), r)
    assert abs(st["E1"] - 4e-4) < 1e-9


def test_uniform_relative_error_above_e1_fails():
    r = _ref()
    with pytest.raises(AssertionError):
        tolerance.check_e1_e2(r * (1 + 2e-3), r)


def test_planted_outlier_fails_e2():
    r = _ref()
    y = r.copy()
    y[7, 9] += 0.05 + 0.006 * abs(r[7, 9])
    with pytest.raises(AssertionError):
        tolerance.check_e1_e2(y, r)


def test_near_zero_absolute_clause():
    r = np.zeros((4, 4))
    y = r + 0.019
    tolerance.check_e2(y, r)
    with pytest.raises(AssertionError):
        tolerance.check_e2(r + 0.021, r)


def test_nonfinite_fails():
    r = _ref()
    y = r.copy()
    y[0, 0] = np.nan
    with pytest.raises(AssertionError):
        tolerance.check_e1_e2(y, r)


def test_e3_cast_check():
    o32 = np.random.default_rng(22).standard_normal((8, 32)).astype(np.float32)
    tolerance.check_e3(codecs.bf16_bits(o32.astype(np.float64)), o32, "bf16")
    tolerance.check_e3(codecs.f16_bits(o32.astype(np.float64)), o32, "f16")
    bad = codecs.bf16_bits(o32.astype(np.float64))
    bad[3, 3] ^= 1
    with pytest.raises(AssertionError):
        tolerance.check_e3(bad, o32, "bf16")
