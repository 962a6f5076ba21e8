"""Seeded synthetic inputs for the routed-attention path.

This package only draws inputs (tensors, overlap matrices, coverage flags).
It holds none of the method's arithmetic and is shared by the tests, the
benchmark and the oracle checks; neither the oracle nor the HIP path imports
the other through it.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .generate import Inputs, make_inputs, bf16_bits_to_f32, f32_to_bf16_bits  # noqa: F401
