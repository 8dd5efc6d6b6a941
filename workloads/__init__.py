"""Seeded synthetic inputs for MLA decode / verify (shared by tests, bench and smoke).

This package only draws random numbers and lays them out; it holds none of
the attention arithmetic.  Both the HIP path and the float64 oracle consume
exactly the bytes produced here.
"""

from .mla_inputs import (
    CONFIGS,
    MLAInputs,
    make_inputs,
    make_config,
    make_c5_layer,
    compact_for_oracle,
    algorithmic_bytes,
    algorithmic_flops,
    SOFTMAX_SCALE,
)

__all__ = [
    "CONFIGS",
    "MLAInputs",
    "make_inputs",
    "make_config",
    "make_c5_layer",
    "compact_for_oracle",
    "algorithmic_bytes",
    "algorithmic_flops",
    "SOFTMAX_SCALE",
]
