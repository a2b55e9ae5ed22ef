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
// r = 256 y + t / 32 + 8 i and adds them in increasing i; the 8 row groups
// are then added in group order through LDS into part[y][col] (fp32). The
// loads of 8 consecutive i are issued before their adds, so that each
// thread has 8 in flight rather than one (the adds keep their order).
template <class S>
__global__ __launch_bounds__(256) void colsum_part_kernel(const typename S::T* __restrict__ m, int64_t rows,
                                                          int64_t cols, float* __restrict__ part) {
  __shared__ float red[8][256];
  const int t = threadIdx.x, cc = t & 31, rg = t >> 5;
  const int64_t c0 = (int64_t)blockIdx.x * 256 + cc * 8;
  const int64_t r0 = (int64_t)blockIdx.y * 256, r1 = min(rows, r0 + 256);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const uint4& w) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += S::to_f((typename S::T)(u[i] & 0xffffu));
      acc[2 * i + 1] += S::to_f((typename S::T)(u[i] >> 16));
    }
  };
  if (c0 < cols) {
    int64_t r = r0 + rg;
    for (; r + 56 < r1; r += 64) {
      uint4 w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = *reinterpret_cast<const uint4*>(m + (r + 8 * j) * cols + c0);
#pragma unroll
      for (int j = 0; j < 8; ++j) add(w[j]);
    }
    for (; r < r1; r += 8) add(*reinterpret_cast<const uint4*>(m + r * cols + c0));
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

// Sum over blocks of part[b][c] in block order, with 8 loads in flight.
__device__ __forceinline__ float colsum_blocks(const float* __restrict__ part, int nblk, int64_t cols, int64_t c) {
  float s = 0.0f;
  int b = 0;
  for (; b + 8 <= nblk; b += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = part[(int64_t)(b + j) * cols + c];
#pragma unroll
    for (int j = 0; j < 8; ++j) s += v[j];
  }
  for (; b < nblk; ++b) s += part[(int64_t)b * cols + c];
  return s;
}

// Second pass: out[c] = round(sum over blocks of part[b][c]) in block order.
template <class S>
__global__ __launch_bounds__(256) void colsum_finish_kernel(const float* __restrict__ part, int nblk, int64_t cols,
                                                            typename S::T* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  out[c] = S::from_f(colsum_blocks(part, nblk, cols, c));
}

// Second pass added to an fp32 buffer (beta = 1): out[c] += sum over blocks
// of part[b][c] in block order.
static __global__ __launch_bounds__(256) void colsum_accum_kernel(const float* __restrict__ part, int nblk,
                                                                 int64_t cols, float* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  out[c] += colsum_blocks(part, nblk, cols, c);
}

}  // namespace tpmlp
