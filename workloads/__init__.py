"""Seeded synthetic inputs for tree-indexed sparse decode attention.

This package only draws random tensors and lays them out. It holds none of the
method's arithmetic (no pooling, scoring, selection or attention), so both the
CPU oracle and the HIP path can consume its output without sharing any code
with each other.
"""

from .synth import (  # noqa: F401
    WORKLOADS,
    spec,
    gen_R,
    gen_Q,
    gen_KV_unit,
    needle_plan,
    gen_all,
    to_storage,
)
