"""CPU oracle for one tensor-parallel rank's share of a Transformer MLP
block and of its self-attention block.

TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check in __graft_entry__
and the cpu_baseline leg of bench.py may import this package; the product
path (the HIP library and its Python binding) never calls it and shares no
code with it.

Everything here is plain float64 NumPy: the unsharded MLP and attention
forward and backward written out from their definitions, shard slicing, and
sampled restrictions of the same definitions for full-size spot checks.
"""
from .attn import (
    attn_forward,
    attn_backward,
    attn_shard_columns,
    attn_shard_weights,
    attn_shard_forward,
    attn_shard_backward,
    row_logsumexp,
    softmax_rows,
    split_heads,
)
from .mlp import (
    GELU_C,
    bias2_grad,
    SQRT_2_OVER_PI,
    gelu,
    gelu_grad,
    mlp_forward,
    mlp_backward,
    shard_weights,
    shard_forward,
    shard_backward,
    reduce_partials,
    sampled_rows,
    sampled_cols,
    rel_err,
)

__all__ = [
    "attn_forward",
    "attn_backward",
    "attn_shard_columns",
    "attn_shard_weights",
    "attn_shard_forward",
    "attn_shard_backward",
    "row_logsumexp",
    "softmax_rows",
    "split_heads",
    "GELU_C",
    "bias2_grad",
    "SQRT_2_OVER_PI",
    "gelu",
    "gelu_grad",
    "mlp_forward",
    "mlp_backward",
    "shard_weights",
    "shard_forward",
    "shard_backward",
    "reduce_partials",
    "sampled_rows",
    "sampled_cols",
    "rel_err",
]
