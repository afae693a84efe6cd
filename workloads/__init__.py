"""Seeded synthetic inputs for prefix-tree-packed attention.

This package only draws inputs: token sequences, segment tables of hand-described
rows and Q/K/V tensors. It holds none of the method's arithmetic (no radix build,
no packing, no mask, no attention) so that both the CPU oracle and the GPU path
can take their inputs from it without sharing any logic.
"""
from .gen import (  # noqa: F401
    CONFIG_NAMES,
    RowInputs,
    SeqBatch,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    make_config,
    config4_sequences,
    GdnInputs,
    draw_gdn,
    draw_grad,
    draw_qkv,
    fill_pads,
    random_forest_row,
    random_sequences,
)
