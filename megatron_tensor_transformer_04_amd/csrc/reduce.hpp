// Sum of P row-parallel partials plus an optional bias over a range of rows:
// the arithmetic of the tensor-parallel all-reduce that follows the second
// linear ("Understanding the Megatron-LM architecture: how 3D parallelism
// assigns roles", section 1, the row-split item: the result of a row split
// is all-reduced), and of the reduce-scatter that replaces it when the
// sequence dimension is split too ("Training GPT-2 with Megatron-LM",
// section 5.1, the --sequence-parallel switch), for P partials held on one
// device.
//
//   out[r][c] = round( sum_{i < P} part_i[row0 + r][c]  (+ bias[c]) )
//
// fp32 sums in rank order, the bias added last, one rounding. HBM-bound:
// each thread moves 16-byte chunks, P loads in flight at once.
#pragma once

#include "numerics.hpp"

namespace tpmlp {

constexpr int kMaxParts = 16;

struct PartList {
  const void* p[kMaxParts];
};

template <class S>
__global__ __launch_bounds__(256) void reduce_partials_kernel(PartList parts, int nparts,
                                                              const typename S::T* __restrict__ bias, int64_t row0,
                                                              int64_t rows, int64_t cols,
                                                              typename S::T* __restrict__ out) {
  using T = typename S::T;
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte chunk
  const int64_t cpr = cols / E;      // chunks per row
  const int64_t total = rows * cpr;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total; q += stride) {
    const int64_t r = q / cpr, c = (q % cpr) * E;
    const int64_t src = (row0 + r) * cols + c;
    u32x4 v[kMaxParts];
#pragma unroll
    for (int i = 0; i < kMaxParts; ++i)
      if (i < nparts) v[i] = *reinterpret_cast<const u32x4*>(static_cast<const T*>(parts.p[i]) + src);
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxParts; ++i) {
      if (i < nparts) {
        const T* x = reinterpret_cast<const T*>(&v[i]);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += S::to_f(x[e]);
      }
    }
    if (bias) {
      const u32x4 b = *reinterpret_cast<const u32x4*>(bias + c);
      const T* x = reinterpret_cast<const T*>(&b);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += S::to_f(x[e]);
    }
    u32x4 o;
    T* y = reinterpret_cast<T*>(&o);
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = S::from_f(acc[e]);
    *reinterpret_cast<u32x4*>(out + r * cols + c) = o;
  }
}

}  // namespace tpmlp
