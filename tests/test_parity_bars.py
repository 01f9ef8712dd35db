"""CPU checks of the comparison helper the GPU tests use (tests/parity.py): each bar
fails where it should, so a green GPU run means what the bars say."""

import numpy as np
import pytest
import torch

from parity import TOL_BF16_ABS, bf16_ulps, check

BF = torch.bfloat16


def test_plain_bf16_bars():
    ref = np.linspace(-2.0, 2.0, 1001)
    ref[7] = np.nan  # entries the oracle did not compute are skipped
    one = np.zeros_like(ref)
    one[3] = 1.0
    check("ok", np.where(np.isnan(ref), 7.0, ref + 0.019 * one), ref, BF)
    with pytest.raises(AssertionError, match="max-abs"):
        check("abs", ref + 0.021 * one, ref, BF)
    with pytest.raises(AssertionError, match="rel-L2"):
        check("rel", ref * 1.006, ref, BF)
    bad = ref.copy()
    bad[5] = np.nan
    with pytest.raises(AssertionError, match="non-finite"):
        check("nan", bad, ref, BF)


def test_lse_and_f32_bars():
    ref = np.array([1.0, 3.0])
    check("lse", ref + 9e-4, ref, BF, lse=True)
    with pytest.raises(AssertionError):
        check("lse", ref + 1.1e-3, ref, BF, lse=True)
    check("f32", ref + 9e-6, ref, torch.float32)
    with pytest.raises(AssertionError):
        check("f32", ref + 1.1e-5, ref, torch.float32)


def test_out_ulp_bar_applies_on_top_of_rounding_only_for_large_values():
    ref = np.array([1.0, 5.0, 9.0, 3.9, np.nan])
    # 9 + 0.035: 0.035 - 9 / 512 = 0.0174 <= 2e-2 on top of the output's rounding
    check("large", np.array([1.01, 5.02, 9.035, 3.9, 0.0]), ref, BF, out_ulp=True)
    # beyond the bar on top of rounding
    with pytest.raises(AssertionError, match="2\\^-9"):
        check("large", np.array([1.0, 5.0, 9.04, 3.9, 0.0]), ref, BF, out_ulp=True)
    # |ref| < 4: 0.0255 - 3.9 / 512 = 0.0179 passes the relaxed form but not the plain bar
    with pytest.raises(AssertionError, match="where \\|ref\\| < 4"):
        check("small", np.array([1.0, 5.0, 9.0, 3.9255, 0.0]), ref, BF, out_ulp=True)


def test_bf16_ulps():
    # spacing of bf16 at 1.0 is 2^-7, at 9.0 it is 2^-4
    assert bf16_ulps(np.array([1.0 + 2.0 ** -7]), np.array([1.0])) == pytest.approx(1.0)
    assert bf16_ulps(np.array([9.0 + 2.0 ** -5]), np.array([9.0])) == pytest.approx(0.5)
    assert TOL_BF16_ABS == 2e-2


def test_out_ulp_bar_with_a_rounded_reference():
    """A reference that is itself a sum of rounded outputs keeps only the
    rounding-aware bar."""
    ref = np.full(1000, 3.0)
    ref[0], ref[1] = 3.9, np.nan
    got = np.where(np.isnan(ref), 0.0, ref)
    got[0] = 3.9255  # 0.0255 - 3.9 / 512 = 0.0179 on top of the rounding
    check("rounded ref", got, ref, BF, out_ulp=True, exact_ref=False)
    with pytest.raises(AssertionError, match="where \\|ref\\| < 4"):
        check("exact ref", got, ref, BF, out_ulp=True)


def test_out_ulp_bar_with_a_gain():
    """A gradient mapped through a map of gain g: the 2e-2 parts of the bar scale by g
    per element, the output's rounding part does not."""
    ref = np.full(1000, 2.0)
    ref[1] = np.nan
    got = np.where(np.isnan(ref), 0.0, ref)
    got[0] = 2.035  # 0.035 > 2e-2, but within 2e-2 * 1.8
    gain = np.ones_like(ref)
    gain[0] = 1.8
    check("gain", got, ref, BF, out_ulp=True, gain=gain)
    with pytest.raises(AssertionError, match="over the gain"):
        check("gain", got, ref, BF, out_ulp=True, gain=np.where(gain > 1, 1.7, 1.0))
    with pytest.raises(AssertionError, match="2\\^-9"):
        check("no gain", got, ref, BF, out_ulp=True)
    with pytest.raises(AssertionError, match="gain below 1"):
        check("gain", got, ref, BF, out_ulp=True, gain=np.full_like(ref, 0.5))
