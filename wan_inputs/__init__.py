"""Seeded synthetic workloads shared by the oracle and the GPU harness (no model arithmetic)."""
from .configs import CONFIGS, WanConfig, get_config, param_count, weight_dtype, weight_spec  # noqa: F401
from .generate import (  # noqa: F401
    ROOT_SEED,
    Tensor,
    Weights,
    bf16_bits_to_f32,
    draw_image,
    draw_inputs,
    draw_latent,
    draw_normal,
    draw_text,
    draw_timestep,
    draw_uniform,
    f32_to_bf16_bits,
)
