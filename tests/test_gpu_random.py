"""GPU parity on seeded random problems (tests/random_cases.py): video tiles
with valid counts, top-k and gate forms, plain sequences with ragged blocks,
packed TND sequences; random block shapes, head groupings, head dimensions,
dtypes and backward variants. Each runs through the C ABI and is compared with
the oracle to the fixed cases' bars, the top-k selection exactly."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import check
from tests.random_cases import N_CASES, describe, random_case

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the CPU container collects but skips these
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.gpu_run import run_case  # noqa: E402
from tests.test_gpu_parity import _compare_case, _topk_agreement  # noqa: E402


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_problem(i):
    case, opts = random_case(i)
    print(describe(case, opts), flush=True)
    res = run_case(case, **opts)
    orc = oracle.Oracle(case, np.float32, threads=16)
    if case.topk > 0:
        assert _topk_agreement(orc, res["map"]).all(), "top-k near-tie"
    _compare_case(case, res, orc)
    if case.gate_mode == "projected":
        check("gate", orc.gate_values(), res["gate_vals"], (2e-3, 1e-2))
