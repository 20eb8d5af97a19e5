"""Seeded synthetic inputs for packed shared-prefix attention.

This package only draws lengths and random tensors. It holds none of the
attention method's arithmetic, so both the fp64 CPU oracle (``oracle/``) and
the HIP path (``shared_prefix_packed_amd``) can take their inputs from it
without sharing any computation.
"""
from .synth import (  # noqa: F401
    Workload,
    WORKLOAD_NAMES,
    make_workload,
    make_custom,
    draw_tensor,
    draw_qkv,
    draw_decode,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    sha256,
)
