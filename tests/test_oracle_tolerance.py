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


def test_e3_rejects_nan_in_both_outputs():
    # An output tile that was never written keeps its NaN fill in both the fp32 and the
    # 16-bit call; equal bit patterns must not make that pass.
    o32 = np.random.default_rng(23).standard_normal((8, 32)).astype(np.float32)
    o32[2, 5] = np.nan
    for kind, bits in (("bf16", codecs.bf16_bits), ("f16", codecs.f16_bits)):
        b = bits(o32.astype(np.float64))
        assert np.isnan(o32[2, 5])
        with pytest.raises(AssertionError, match="non-finite"):
            tolerance.check_e3(b, o32, kind)


def test_e3_rejects_nan_in_16bit_output_only():
    o32 = np.random.default_rng(24).standard_normal((8, 32)).astype(np.float32)
    b = codecs.f16_bits(o32.astype(np.float64))
    b[1, 1] = 0x7E00                                    # fp16 quiet NaN
    with pytest.raises(AssertionError, match="non-finite"):
        tolerance.check_e3(b, o32, "f16")


def test_combined_chunk_statistics_equal_whole():
    r = _ref()
    y = r * (1 + 3e-4)
    y[40, 3] += 0.01
    whole = tolerance.error_stats(y, r)
    parts = [tolerance.error_stats(y[i:i + 16], r[i:i + 16]) for i in range(0, 64, 16)]
    comb = tolerance.combine_stats(parts)
    assert abs(comb["E1"] - whole["E1"]) <= 1e-15 * whole["E1"] + 1e-18
    for k in ("E2_worst_ratio", "max_abs", "max_rel_big", "E2_fail_count", "nonfinite", "count"):
        assert comb[k] == whole[k], k
    assert tolerance.gates_pass(comb)
    y[5, 5] = np.inf
    assert not tolerance.gates_pass(tolerance.combine_stats([tolerance.error_stats(y, r)]))


def test_max_relative_error_over_typical_magnitudes():
    # 1% error on one element of typical size shows in max_rel_rms although it passes E2's
    # absolute clause; a 1% error on a near-zero element does not count there.
    r = np.array([[3.0, -2.5, 1e-3, 2.8]])
    y = r.copy()
    y[0, 0] *= 1.01
    st = tolerance.error_stats(y, r)
    assert abs(st["max_rel_rms"] - 0.01) < 1e-12
    y = r.copy()
    y[0, 2] *= 1.01
    assert tolerance.error_stats(y, r)["max_rel_rms"] == 0.0
