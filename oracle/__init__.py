"""CPU oracle for one tensor-parallel rank's share of a Transformer MLP.

TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check in __graft_entry__
and the cpu_baseline leg of bench.py may import this package; the product
path (the HIP library and its Python binding) never calls it and shares no
code with it.

Everything here is plain float64 NumPy: the unsharded MLP forward and
backward written out from their definitions, shard slicing, and sampled
restrictions of the same definitions for full-size spot checks.
"""
from .mlp import (
    GELU_C,
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
    "GELU_C",
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
