// The MLP shard's GEMM planner and engines, as used by the attention shard
// built into the same library (its four projections and their gradients).
//
// C[M][N] (16-bit, row pitch ldo) = sum_k P[m][k] Q[k][n], plus bias[n] when
// bias is not null, rounded once. pk / qk: P / Q k-contiguous (P[m][k] at
// p[m ldp + k], Q[k][n] at q[n ldq + k]) or mn-contiguous (p[k ldp + m],
// q[k ldq + n]). The planner picks the engine and tile as for the MLP's own
// GEMMs; a plain store (no bias) may split k into fp32 partials at tail_ws
// when planned_gemm_tail_bytes(...) of them fit in tail_cap.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tpmlp {

hipError_t planned_gemm(int dtype, bool pk, bool qk, int64_t M, int64_t N, int64_t K, const void* p, int64_t ldp,
                        const void* q, int64_t ldq, void* out, int64_t ldo, const void* bias, float* tail_ws,
                        size_t tail_cap, hipStream_t st);

// Bytes of fp32 k-split partials a plain-store planned_gemm of this shape
// uses (0 if it splits nothing); kc: both operands k-contiguous.
size_t planned_gemm_tail_bytes(int dtype, int64_t M, int64_t N, int64_t K, bool kc);

// Does a GEMM of this shape run on the large-tile direct-load engine once
// both operands are k-contiguous (so that staging a transposed copy of an
// mn-contiguous operand pays off)?
bool planned_gemm_stages(int dtype, int64_t M, int64_t N, int64_t K);
// The same for a GEMM whose mn-contiguous operand is a weight, which is
// also copied where the copy buys the 16x16 MFMA form (256 x 256 tiles).
bool planned_gemm_stages_weight(int dtype, int64_t M, int64_t N, int64_t K);

// out[c][r] = in[r][c] for a dense 16-bit [R][C] matrix; out has row pitch
// staged_transpose_ld(R) (R plus padding that spreads its rows over the L2
// channels).
hipError_t staged_transpose(const void* in, void* out, int64_t R, int64_t C, hipStream_t st);
int64_t staged_transpose_ld(int64_t R);

}  // namespace tpmlp
