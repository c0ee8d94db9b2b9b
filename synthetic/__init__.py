"""Seeded synthetic inputs (random draws and bf16 bit packing only)."""
from .gen import *  # noqa: F401,F403
from .gen import (ROW_BLOCK, Walk, activation_walk, activations, heads_walk, bf16_bits_to_f32, f32_to_bf16_bits, heads_activations,  # noqa: F401
                  mlp_weights, scores, stream, walk_block, weight)
