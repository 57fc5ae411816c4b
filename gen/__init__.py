"""Seeded synthetic inputs for the expert-parallel layout / dispatch / combine path.

This package only draws random numbers and arranges them into the input
tensors (token rows, top-k expert ids, top-k weights).  It holds none of the
routing, packing or reduction arithmetic, so both the CPU oracle and the HIP
path can consume the same inputs without sharing any method code.
"""

from .inputs import (  # noqa: F401
    CONFIGS,
    Inputs,
    config_inputs,
    generate,
    random_case,
    random_rows,
)
