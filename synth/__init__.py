"""Seeded synthetic inputs for the Dual-AR decode path.

This package generates *data only*: model hyper-parameters of the five
workloads, random-init weights, prompts, top-p uniforms and context lengths.
It holds none of the method's arithmetic (no embedding, attention, norm or
sampling code), so both the CPU oracle and the HIP path may consume it.
"""
from .inputs import (  # noqa: F401
    MODELS,
    WORKLOADS,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_ctx_lengths,
    make_fast_inputs,
    make_prompts,
    make_uniforms,
    make_weights,
    model,
    prompt_lengths,
    tensor_specs,
    W4_GROUP,
    make_w4_model,
    quantize_w4,
    w4_names,
    weights_as_f32,
)
