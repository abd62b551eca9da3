"""Seeded synthetic inputs for the gpt-oss MoE FFN layer.

This package is shared by the tests, the bench and the smoke check. It only
draws and encodes inputs (random bf16 activations, fp32 router parameters,
random MXFP4 code and scale bytes, bf16 biases). It holds none of the layer's
arithmetic: no routing, no dequantisation, no matrix product of the layer.
"""
from .gen import (  # noqa: F401
    H_DEFAULT,
    I_DEFAULT,
    LAYER_CONFIGS,
    LayerConfig,
    bf16_bits_from_f32,
    device_activations,
    make_layer_inputs,
    make_config_inputs,
    zipf_target_shares,
)
