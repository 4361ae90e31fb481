"""Seeded synthetic inputs for one layer's compressed sparse attention step.

This package only draws random numbers and rounds them to their stored
dtypes.  It holds none of the method's arithmetic, so the CPU oracle and the
HIP path can both consume its arrays without sharing any computation.
"""
from .inputs import CONFIGS, Workload, make_config, make_unit, bf16_bits_from_f32, f16_bits_from_f32  # noqa: F401
