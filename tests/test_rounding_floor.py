"""The rounding floor that sets the avg_abs bar of large 16-bit results
(tests/helpers.py): it is the mean error of one round-to-nearest-even to the
output type, so it vanishes on representable values, sits near a quarter of
the unit in the last place on average, and raises the bar only for tensors
whose entries are large."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from tests.helpers import FLOOR_FACTOR, GRAD_TOL, check, rounding_floor


@pytest.mark.parametrize("dtype, mant", [("bf16", 8), ("fp16", 11)])
def test_floor_is_zero_on_representable_values_and_a_quarter_ulp_on_average(dtype, mant):
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    rng = np.random.default_rng(3)
    exact = torch.from_numpy(rng.uniform(1.0, 2.0, 20000)).to(tdt).double().numpy()
    assert rounding_floor(exact, dtype) == 0.0
    # uniform on [1, 2): spacing 2^(1 - mant), mean rounding error a quarter of it
    x = rng.uniform(1.0, 2.0, 200000)
    assert rounding_floor(x, dtype) == pytest.approx(2.0 ** (1 - mant) / 4, rel=0.02)


def test_bar_rises_only_for_large_tensors():
    rng = np.random.default_rng(4)
    small = rng.normal(0.0, 0.1, 4096)
    big = rng.normal(0.0, 3.0, 4096)
    assert FLOOR_FACTOR * rounding_floor(small, "bf16") < GRAD_TOL[0]
    assert FLOOR_FACTOR * rounding_floor(big, "bf16") > GRAD_TOL[0]
    # a result off by 1 % everywhere fails either way; one off by a single
    # bf16 rounding passes the raised bar for the large tensor
    with pytest.raises(AssertionError):
        check("big", big, big * 1.01, GRAD_TOL, "bf16")
    rounded = torch.from_numpy(big).to(torch.bfloat16).double().numpy()
    check("big", big, rounded, GRAD_TOL, "bf16")
    with pytest.raises(AssertionError):
        check("big", big, rounded, GRAD_TOL)
