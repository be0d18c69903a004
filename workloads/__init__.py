"""Seeded synthetic inputs for block-sparse attention.

This package only draws random tensors, masks and lengths with the shapes and
distributions of the workloads on the source pages. It computes nothing of the
attention method itself, so both the HIP path and the CPU oracle may use it.
"""

from .synth import Case, CASES, make_case, vsa_tile_counts  # noqa: F401
