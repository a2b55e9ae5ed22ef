// fp32 GEMM engine with plain fp32 fused multiply-adds (no reduced-precision
// matrix mode): C[M][N] = sum_k P[m][k] Q[k][n] with the same operand layouts
// (KC / MC) and epilogues as the MFMA engine. It serves fp32 storage, whose
// tolerance needs true fp32 products; 64x64 tiles, 256 threads, each thread
// owning a strided 4x4 block of outputs, K staged 16 at a time through LDS.
#pragma once

#include "gemm_mfma.hpp"
#include "numerics.hpp"

namespace tpmlp {

struct SimtTile {
  static constexpr int BM = 64, BN = 64, BK = 16, THREADS = 256, GROUP = 8;
};

struct OperandF32 {
  const float* ptr;
  int64_t ld;
};

template <bool KC>
__device__ __forceinline__ float load_f32(const OperandF32& op, int64_t mn, int64_t MN, int64_t k, int64_t kend) {
  if (mn < MN && k < kend) return KC ? op.ptr[mn * op.ld + k] : op.ptr[k * op.ld + mn];
  return 0.0f;
}

template <bool P_KC, bool Q_KC, bool GELU_P, class Epi>
__global__ __launch_bounds__(256) void gemm_simt_kernel(GemmShape sh, OperandF32 P, OperandF32 Q, Epi epi) {
  constexpr int BM = SimtTile::BM, BN = SimtTile::BN, BK = SimtTile::BK;
  __shared__ float sP[BK][BM + 1];
  __shared__ float sQ[BK][BN + 1];
  __shared__ float red[16][BN];

  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  int split, tm, tn;
  map_tile<SimtTile::GROUP>(blockIdx.x, gridDim.x, sh.tiles_m, sh.tiles_n, split, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t kbeg = (int64_t)split * sh.k_per;
  const int64_t kend = min(sh.K, kbeg + sh.k_per);

  float acc[4][4] = {};
  for (int64_t k0 = kbeg; k0 < kend; k0 += BK) {
    // 64 x 16 elements per operand, four per thread
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = tid + c * 256;
      // KC: 16 consecutive k per row; MC: 64 consecutive rows per k
      const int mn = P_KC ? (e >> 4) : (e & 63), kk = P_KC ? (e & 15) : (e >> 6);
      float v = load_f32<P_KC>(P, m0 + mn, sh.M, k0 + kk, kend);
      if constexpr (GELU_P) v = gelu_tanh(v);
      sP[kk][mn] = v;
      const int mq = Q_KC ? (e >> 4) : (e & 63), kq = Q_KC ? (e & 15) : (e >> 6);
      sQ[kq][mq] = load_f32<Q_KC>(Q, n0 + mq, sh.N, k0 + kq, kend);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sP[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sQ[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

  float cs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty + 16 * i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx + 16 * j;
      if (m < sh.M && n < sh.N) cs[j] += epi.apply(m, n, acc[i][j]);
    }
  }
  if constexpr (Epi::kColSum) {
#pragma unroll
    for (int j = 0; j < 4; ++j) red[ty][tx + 16 * j] = cs[j];
    __syncthreads();
    if (tid < BN) {
      float s = 0.0f;
      for (int r = 0; r < 16; ++r) s += red[r][tid];
      if (n0 + tid < sh.N) epi.colsum(tm, n0 + tid, s);
    }
  }
}

}  // namespace tpmlp
