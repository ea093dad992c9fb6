"""CPU pins of the FP8 quantisation floors (tests/fp8_cases.py, tests/golden/fp8_quantisation_floors.txt).

The FP8 bar is O RMSE <= 3e-2 against fp64 on the unquantised inputs.  For the cases below, exact
fp64 attention on the e4m3-dequantised inputs -- computed here from the oracle alone -- already
misses that bar, so no implementation of the method (power-of-two scales per 64 x d block, e4m3
codes) can meet it there; the GPU tests hold the kernel to the stored floor plus its own error
allowance.  This test recomputes each floor, checks it against the stored value, and checks that
each one does exceed the bar (otherwise the plain bar would apply).  The independent-channel
reading of the FP8 workload's outliers stays below the bar, and is held to it."""
import numpy as np
import pytest

import seeded_inputs as si
from tests import fp8_cases

BAR = 3e-2


@pytest.mark.parametrize("name", fp8_cases.CASES)
def test_floor_matches_stored_value_and_exceeds_bar(name):
    stored = fp8_cases.stored_floors()[name]
    m = fp8_cases.quantisation_floor(*fp8_cases.case(name))
    assert m["rmse"] == pytest.approx(stored, rel=1e-12, abs=0.0), (name, m, stored)
    assert m["rmse"] > BAR, f"{name}: floor {m['rmse']:.4g} is under the bar; the plain bar applies"


def test_fp8_workload_floor_value():
    """The FP8 workload (two x20 outlier channels shared by Q, K and V): the floor is 0.0357, the
    figure the kernel is compared with (it measures about 0.036)."""
    assert fp8_cases.stored_floors()["c5_shared_channels"] == pytest.approx(0.03569, abs=1e-5)


def test_independent_channel_reading_is_under_the_bar():
    """The other reading of the outlier construction (independent channel draws for Q, K and V):
    its floor is well under 3e-2, so the GPU test holds the kernel to 3e-2 itself."""
    inp = si.fp8_inputs(2, 8192, 16, 128, seed=5, independent_channels=True)
    heads, tokens = fp8_cases.sample_rows(inp, 2048, seed=2)
    m = fp8_cases.quantisation_floor(inp, si.hadamard_signs(128, seed=55), heads, tokens)
    assert m["rmse"] < BAR / 2, m
