"""Seeded synthetic inputs for KDA prefill and decode and the short conv.

This package only draws random numbers and rounds them to storage dtypes.  It
holds none of the attention arithmetic, so the CPU oracle and the HIP path can
both consume its output without sharing any of the method.
"""
from .kda_inputs import (  # noqa: F401
    CONFIGS,
    KdaInputs,
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    make_config,
    make_inputs,
    seeded_lengths,
    slice_heads,
)
from .conv_inputs import ConvInputs, make_conv_inputs, seeded_conv_lengths  # noqa: F401
