"""The FP8 code checker's acceptance rules, on hand-made codes (no GPU, no kernel output).

A code one step from the oracle's passes only on a rounding boundary; a code several steps off
passes only with LayerNorm's cancellation allowance (`slack`, in scaled units), when its value
lies within that allowance plus one code spacing of the exact scaled value. E5M2 near zero is
where the allowance spans several codes.
"""
import numpy as np
import pytest

import checks
from oracle import formats as F

E5 = F.FORMATS["e5m2"]


def _codes(vals):
    return np.array([F.fp8_encode(np.float64(v), E5) for v in vals], np.uint8)


def test_identical_codes_pass():
    u = np.array([4.8e-4, 1.0, -3.0])
    c = _codes(u)
    assert checks.check_fp8(c, c, u, "e5m2", check_fraction=False)["differ"] == 0


def test_multi_step_code_needs_the_allowance():
    u = np.full(4000, 0.25)
    u[0] = 2.0 ** -11                      # exact scaled value near zero
    ref = _codes(u)
    got = ref.copy()
    got[0] = _codes([1.25 * 2.0 ** -13])[0]  # several E5M2 steps below
    with pytest.raises(AssertionError, match="more than one step"):
        checks.check_fp8(got, ref, u, "e5m2", check_fraction=False)
    slack = np.zeros_like(u)
    slack[0] = 0.02                        # 2^-21 * terms at a block exponent of -14
    rep = checks.check_fp8(got, ref, u, "e5m2", slack=slack, check_fraction=False)
    assert rep["differ"] == 1 and rep["slack"] == 1


def test_multi_step_code_outside_the_allowance_fails():
    u = np.full(4000, 0.25)
    u[0] = 2.0 ** -11
    ref = _codes(u)
    got = ref.copy()
    got[0] = _codes([2.0 ** -6])[0]        # 0.0156 away: beyond a 1e-3 allowance
    slack = np.zeros_like(u)
    slack[0] = 1e-3
    with pytest.raises(AssertionError, match="more than one step"):
        checks.check_fp8(got, ref, u, "e5m2", slack=slack, check_fraction=False)
