"""Seeded synthetic inputs for the routed-attention path.

This package only draws inputs (tensors, overlap matrices, coverage flags,
and the synthetic camera geometry of frustum workloads).  It holds none of
the routed layer's arithmetic (pooling, scoring, modulation, selection,
attention).  For frustum workloads it evaluates the overlap of the drawn
geometry once, as workload data; the on-device overlap builder recomputes
that overlap from the same geometry and is checked against the oracle's own
implementation, never against this one.  Neither the oracle nor the HIP path
imports the other through this package.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .generate import (FrustumGeometry, Inputs, bf16_bits_to_f32, draw_frustum_geometry,  # noqa: F401
                       f32_to_bf16_bits, frustum_overlap, make_inputs)
