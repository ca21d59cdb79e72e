"""Seeded synthetic workloads shared by the oracle and the GPU path (inputs only)."""
from .configs import Shape, CONFIGS, MINI, get, with_tokens
from .gen import generate, to_f32, bf16_bits_to_f32, f32_to_bf16_bits_trunc
