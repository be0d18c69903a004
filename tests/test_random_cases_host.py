"""The seeded random problems of the GPU parity test are well formed: each
draws the same case on every call and passes the library's host-side
validation (so the GPU test exercises supported shapes only)."""

from __future__ import annotations


import bwd_block_map_amd as vsa
from tests.gpu_run import device_inputs, problem_for
from tests.random_cases import N_CASES, random_case


def test_random_problems_are_reproducible_and_valid():
    kinds = set()
    for i in range(N_CASES):
        case, opts = random_case(i)
        again, opts2 = random_case(i)
        assert opts == opts2 and torch_equal(case.q, again.q)
        d = device_inputs(case, "cpu")
        vsa.vsa_validate(problem_for(case, d, **opts))
        kinds.add((case.layout, case.topk > 0, case.gate_mode))
    assert len(kinds) >= 8  # the draws span layouts, top-k and gate forms


def torch_equal(a, b):
    return a.shape == b.shape and bool((a == b).all())
