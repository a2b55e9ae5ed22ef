// The MLP shard's launch sequences (and, for 16-bit storage, the planned
// GEMMs of the attention shard) instantiated for StoreF32.
#include "mlp_impl.hpp"

TPMLP_MLP_INSTANCES(, tpmlp::StoreF32)
