// The MLP shard's launch sequences (and, for 16-bit storage, the planned
// GEMMs of the attention shard) instantiated for StoreBF16.
#include "mlp_impl.hpp"

TPMLP_MLP_INSTANCES(, tpmlp::StoreBF16)
TPMLP_GEMM_INSTANCES(, tpmlp::StoreBF16)
