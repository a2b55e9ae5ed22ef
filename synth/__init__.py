"""Seeded synthetic inputs for the tensor-parallel MLP shard.

This module is shared by the CPU oracle and by the GPU path's tests and
benchmark. It draws random tensors and rounds them to the storage dtype; it
holds none of the MLP's arithmetic (no GEMM, no GeLU, no gradient).

Workloads follow the model shapes printed on the pages:
  * "Training GPT-2 with Megatron-LM" (devpress.csdn.net), section 4.1 (the
    2.4B run: hidden 2560, seq 2048, micro-batch 4), section 4.2 (GPT-2 117M
    row of the learning-rate table), section 5.1 (the 7B run with TP 4) and
    section 1 (a 4096-dim FFN split into 4 blocks);
  * "Understanding the Megatron-LM architecture: how 3D parallelism assigns
    roles" (tbr8.org), practical example (72 layers, hidden 10240, TP 4,
    micro-batch 8).
Values are i.i.d. Gaussians (no structure), drawn in float64 with NumPy's
PCG64 and rounded to nearest-even into the storage dtype, so that the oracle
and the GPU consume bit-identical operands.
"""
from .configs import ATTN_CONFIGS, CONFIGS, AttnConfig, Config, get_attn_config, get_config, shard_width
from .draw import (
    AttnInputs,
    draw_attn_inputs,
    draw_config,
    Inputs,
    draw_inputs,
    round_to_storage,
    storage_bits,
    STORAGE_NUMPY,
)

__all__ = [
    "ATTN_CONFIGS",
    "AttnConfig",
    "AttnInputs",
    "draw_attn_inputs",
    "get_attn_config",
    "CONFIGS",
    "Config",
    "get_config",
    "shard_width",
    "Inputs",
    "draw_inputs",
    "draw_config",
    "round_to_storage",
    "storage_bits",
    "STORAGE_NUMPY",
]
