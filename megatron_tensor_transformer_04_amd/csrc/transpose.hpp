// out[c][r] = in[r][c] for a dense row-major [R][C] matrix of 16-bit values
// (R and C multiples of 8); out rows are ldo >= R elements apart (ldo a
// multiple of 8; columns R..ldo-1 are not written).
//
// The large-tile GEMM engine reads k-contiguous operands fastest (one
// ds_read_b128 per fragment; an mn-contiguous operand needs two transposing
// reads per fragment, for every wave that uses it). Operands stored
// mn-contiguous are therefore transposed once, by this HBM-bound kernel,
// into caller workspace before the GEMM that reads them.
//
// Each lane moves one 8 x 8 block entirely in registers: eight 16-byte loads
// (eight rows of eight columns), 32 byte permutes, eight 16-byte stores
// (eight output rows of eight columns). A wave covers a 64 x 64 tile with
// lane l on block row l / 8 and block column l % 8, so every load
// instruction reads eight 128-byte row segments and every store writes
// eight 128-byte output-row segments. No LDS.
//
// With GELU, each value is replaced by rne(gelu(value)) on the way (the
// backward's H^T when the forward did not keep H).
#pragma once

#include "numerics.hpp"

namespace tpmlp {

constexpr int kTrWaveTile = 64;            // rows and columns per wave
constexpr int kTrWaves = 4;                // waves per workgroup, side by side along C
constexpr int kTrCols = kTrWaveTile * kTrWaves;

template <class S, bool GELU>
__global__ __launch_bounds__(64 * kTrWaves) void transpose16_kernel(const uint16_t* __restrict__ in,
                                                                    uint16_t* __restrict__ out, int64_t R, int64_t C,
                                                                    int64_t ldo, int tiles_c) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tr = blockIdx.x / tiles_c, tc = blockIdx.x % tiles_c;
  const int64_t r = (int64_t)tr * kTrWaveTile + (lane >> 3) * 8;                 // first row of the block
  const int64_t c = (int64_t)tc * kTrCols + wave * kTrWaveTile + (lane & 7) * 8;  // first column
  if (r >= R || c >= C) return;
  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = *reinterpret_cast<const u32x4*>(in + (r + i) * C + c);
    if constexpr (GELU) v[i] = gelu_chunk<S>(v[i]);
  }
  // Output row c + j holds in[r + i][c + j], i = 0..7: dword w pairs rows
  // 2w (low half) and 2w + 1 (high half); column j sits in dword j / 2 of
  // each input row, low half for even j. v_perm_b32 selectors: bytes
  // 0x05040100 take the low halves of (hi_src, lo_src), 0x07060302 the highs.
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) o[w] = __builtin_amdgcn_perm(v[2 * w + 1][j >> 1], v[2 * w][j >> 1], sel);
    *reinterpret_cast<u32x4*>(out + (c + j) * ldo + r) = o;
  }
}

}  // namespace tpmlp
