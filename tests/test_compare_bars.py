"""The parity bars in oracle/compare.py hold the stated tolerances (CPU only)."""
import math

import numpy as np
import pytest

from oracle import compare as C


def _abc_with_condition(cond):
    """Centred covariance entries (a, b, c) whose condition sqrt((a-b)^2 + 4c^2)/(a+b)
    equals `cond` (a + b = 2)."""
    return np.array([[1.0 + cond / 2, 1.0 - cond / 2, 0.0]])


@pytest.mark.parametrize("cond", [1.0, 1e-3, 1e-5, 1e-7, 2e-9])
def test_angle_bar_never_exceeds_one_microradian(cond):
    """Down to the ill-conditioned cutoff, an error above 1e-6 rad fails, however
    badly conditioned the pair (the summation-order term 1e-11 / cond alone would
    allow up to 5e-3 rad at cond = 2e-9)."""
    abc = _abc_with_condition(cond)
    ref = np.array([0.3])
    bar = min(2.0 ** -25 + 1e-11 / cond, 1e-6)
    C.compare_angles(np.array([0.3 + 0.9 * bar]), ref, abc)
    with pytest.raises(C.ParityError):
        C.compare_angles(np.array([0.3 + 1.5e-6]), ref, abc)


def test_angle_bar_is_one_fp32_rounding_on_well_conditioned_pairs():
    abc = _abc_with_condition(0.5)
    ref = np.array([0.3])
    C.compare_angles(np.array([0.3 + 2.9e-8]), ref, abc)       # below 2^-25 + 2e-11
    with pytest.raises(C.ParityError):
        C.compare_angles(np.array([0.3 + 5e-8]), ref, abc)


def test_only_pairs_below_the_condition_cutoff_are_exempt():
    abc = np.array([[1.0, 1.0, 0.0], [1.0 + 0.5e-9, 1.0 - 0.5e-9, 0.0]])  # cond 0 and 5e-10
    rep = C.compare_angles(np.array([0.4, -0.2]), np.array([0.0, 0.1]), abc)
    assert rep["ill_conditioned"] == 2


def test_angles_compare_modulo_the_quarter_turn_period():
    abc = _abc_with_condition(0.5)
    C.compare_angles(np.array([math.pi / 4 - 1e-9]), np.array([-math.pi / 4]), abc)
