// Fixed-order column sums of a [rows][cols] 16-bit matrix (cols a multiple
// of 8) in two passes: fp32 partial sums per block of 256 rows, then their
// sum in block order, rounded once to the storage dtype or added to an fp32
// buffer. Used for the bias gradients (dbqkv of the attention shard, db2 of
// the MLP block).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "numerics.hpp"

namespace tpmlp {

// Column sums of a [rows][cols] 16-bit matrix (cols a multiple of 8), first
// pass: block (x, y) covers columns [256 x, 256 x + 256) and rows
// [256 y, 256 y + 256). Thread t reads 16-byte chunks (8 columns) of the rows
// r = 256 y + t / 32 + 8 i in order; the 8 row groups are then added in
// group order through LDS into part[y][col] (fp32).
template <class S>
__global__ __launch_bounds__(256) void colsum_part_kernel(const typename S::T* __restrict__ m, int64_t rows,
                                                          int64_t cols, float* __restrict__ part) {
  __shared__ float red[8][256];
  const int t = threadIdx.x, cc = t & 31, rg = t >> 5;
  const int64_t c0 = (int64_t)blockIdx.x * 256 + cc * 8;
  const int64_t r0 = (int64_t)blockIdx.y * 256, r1 = min(rows, r0 + 256);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (c0 < cols) {
    for (int64_t r = r0 + rg; r < r1; r += 8) {
      const uint4 w = *reinterpret_cast<const uint4*>(m + r * cols + c0);
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += S::to_f((typename S::T)(u[i] & 0xffffu));
        acc[2 * i + 1] += S::to_f((typename S::T)(u[i] >> 16));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[rg][cc * 8 + i] = acc[i];
  __syncthreads();
  const int64_t c = (int64_t)blockIdx.x * 256 + t;
  if (c < cols) {
    float v = 0.0f;
#pragma unroll
    for (int g = 0; g < 8; ++g) v += red[g][t];
    part[(int64_t)blockIdx.y * cols + c] = v;
  }
}

// Second pass: out[c] = round(sum over blocks of part[b][c]) in block order.
template <class S>
__global__ __launch_bounds__(256) void colsum_finish_kernel(const float* __restrict__ part, int nblk, int64_t cols,
                                                            typename S::T* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  float s = 0.0f;
  for (int b = 0; b < nblk; ++b) s += part[(int64_t)b * cols + c];
  out[c] = S::from_f(s);
}

// Second pass added to an fp32 buffer (beta = 1): out[c] += sum over blocks
// of part[b][c] in block order.
static __global__ __launch_bounds__(256) void colsum_accum_kernel(const float* __restrict__ part, int nblk,
                                                                 int64_t cols, float* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  float s = 0.0f;
  for (int b = 0; b < nblk; ++b) s += part[(int64_t)b * cols + c];
  out[c] += s;
}

}  // namespace tpmlp
