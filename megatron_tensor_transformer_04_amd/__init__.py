"""MI355X (gfx950) tensor-parallel MLP shard: forward and backward of one
rank's share of a Transformer FFN block, as hand-written HIP kernels behind
the C ABI in include/tp_mlp.h, and of the attention block's share
(include/tp_attn.h). This package is the ctypes binding to that
library (libtpmlp.so, built in-tree by _build.build()).
"""
from ._binding import (  # noqa: F401
    attn_bwd,
    attn_fwd,
    attn_shape,
    tp_attn_bwd,
    tp_attn_bwd_workspace_bytes,
    tp_attn_fwd,
    tp_attn_fwd_workspace_bytes,
    BWD_EVENTS,
    EXPORTS,
    FWD_EVENTS,
    RECOMPUTE_EVENTS,
    LIB_PATH,
    STATUS,
    TPMLP_BF16,
    TPMLP_F16,
    TPMLP_F32,
    TPMLP_LAYOUT_B_T,
    TPMLP_MAX_PARTS,
    TPMLP_WS_DZ,
    TPMLP_WS_MINIMAL,
    TPMLP_WS_RECOMPUTE,
    TpMlpError,
    bwd,
    bwd_recompute,
    fwd,
    load,
    tp_mlp_abi_version,
    tp_mlp_bwd,
    tp_mlp_bwd_main_grad,
    tp_mlp_bwd_recompute,
    tp_mlp_fwd,
    tp_mlp_fwd_workspace_bytes,
    tp_mlp_reduce_partials,
    tp_mlp_status_string,
    tp_mlp_workspace_bytes,
)
