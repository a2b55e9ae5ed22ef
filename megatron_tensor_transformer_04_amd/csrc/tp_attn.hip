// C ABI of the tensor-parallel self-attention shard (declared in
// include/tp_attn.h): one rank's heads, forward and backward.
//
// The projections (QKV, the output projection and their gradients) go
// through the MLP shard's GEMM planner (shard_gemm.hpp): direct-load engine
// with k-split partials where the shapes fill the chip that way. The
// per-head products run on the register-staged MFMA engine (gemm_mfma.hpp,
// 128 x 128 tiles), one batched launch each (scores, P V and the four
// backward products): grid y runs over the
// batch * heads (sequence, head) pairs, and a batched epilogue moves the
// operands and its output to that pair's blocks before the tile is computed.
// Operands are read where they lie (Q, K, V as column blocks of QKV with row
// pitch 3q; O, dO with pitch q): a head's block is k-contiguous or
// mn-contiguous for each product and the engine reads either layout.
//
// Between the products, two row kernels: the fused scale + causal mask +
// softmax over fp32 scores (one wave per row), and its backward
// dS = P * (dP - rowsum(P * dP)) / sqrt(d). dbqkv is a two-pass fixed-order
// column sum.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "tp_attn.h"
#include "attn_common.hpp"
#include "colsum.hpp"
#include "epilogues.hpp"
#include "gemm_mfma.hpp"
#include "shard_gemm.hpp"

namespace tpmlp {
namespace {

using namespace attn;
using CfgA = MfmaTile<128, 128, 2, 2>;

// Offsets (in elements) of batch z = b * inner + j: operand P, operand Q and
// the output each move by b * (stride per sequence) + j * (stride per head).
// `tri` is the causal structure the product can exploit (all of it zero
// when the mask is off):
//   kSkipUpper  outputs [query][key]: tiles whose keys all follow their
//               queries are never read (the softmax and its backward read
//               only keys <= query), so they are not computed;
//   kKeysUpTo   k runs over keys and P[query][key] = 0 for key > query:
//               a tile of queries [m0, m0 + BM) needs keys < m0 + BM only;
//   kQueriesFrom  rows are keys and k runs over queries: P[query][key] = 0
//               for query < key, so a tile of keys [m0, ...) needs queries
//               >= m0 only.
//   kSkipLower  outputs [key][query] (the transposed scores): tiles whose
//               keys all follow their queries are not computed.
enum Tri : int { kNone = 0, kSkipUpper = 1, kKeysUpTo = 2, kQueriesFrom = 3, kSkipLower = 4 };

struct BatchMap {
  int inner;
  int64_t p_b, p_j, q_b, q_j, o_b, o_j;
  int tri;
};

template <int BM, int BN>
__device__ __forceinline__ bool tri_skip(int tri, int64_t m0, int64_t n0) {
  return (tri == kSkipUpper && n0 > m0 + BM - 1) || (tri == kSkipLower && m0 > n0 + BN - 1);
}

template <int BM>
__device__ __forceinline__ void tri_window(int tri, int64_t m0, int64_t& kbeg, int64_t& kend) {
  if (tri == kKeysUpTo) kend = min(kend, m0 + BM);
  if (tri == kQueriesFrom) kbeg = max(kbeg, m0);
}

// Plain store of one (sequence, head) product into its block of a larger
// matrix (row pitch ld), rounded once to the storage dtype.
template <class S>
struct EpiStoreBatched {
  typename S::T* out;
  int64_t ld;
  BatchMap bm;
  static constexpr bool kBatched = true;
  static constexpr bool kColSum = false;
  __device__ __forceinline__ void select(int z, Operand& P, Operand& Q) {
    const int64_t b = z / bm.inner, j = z % bm.inner;
    P.ptr += b * bm.p_b + j * bm.p_j;
    Q.ptr += b * bm.q_b + j * bm.q_j;
    out += b * bm.o_b + j * bm.o_j;
  }
  __device__ __forceinline__ bool skip(int64_t m0, int64_t n0) const {
    return tri_skip<CfgA::BM, CfgA::BN>(bm.tri, m0, n0);
  }
  __device__ __forceinline__ void k_window(int64_t m0, int64_t& kbeg, int64_t& kend) const {
    tri_window<CfgA::BM>(bm.tri, m0, kbeg, kend);
  }
  __device__ __forceinline__ float apply(int64_t m, int64_t n, float acc) const {
    out[m * ld + n] = S::from_f(acc);
    return 0.0f;
  }
  __device__ __forceinline__ void colsum(int, int64_t, float) const {}
};

// Transposed fp32 store of a batched product C [M = keys][N = queries]:
// out[n][m .. m + 3] = C[m .. m + 3][n] as one 16-byte store per lane and
// fragment (the MFMA result gives each lane four consecutive rows of one
// column). Computing the scores (and dP) as K Q^T (V dO^T) with this store
// writes each query's row of keys in 16-byte pieces.
struct EpiStoreF32TBatched {
  float* out;
  int64_t ld;
  BatchMap bm;
  static constexpr bool kBatched = true;
  static constexpr bool kApply4 = true;
  static constexpr bool kColSum = false;
  __device__ __forceinline__ void select(int z, Operand& P, Operand& Q) {
    const int64_t b = z / bm.inner, j = z % bm.inner;
    P.ptr += b * bm.p_b + j * bm.p_j;
    Q.ptr += b * bm.q_b + j * bm.q_j;
    out += b * bm.o_b + j * bm.o_j;
  }
  __device__ __forceinline__ bool skip(int64_t m0, int64_t n0) const {
    return tri_skip<CfgA::BM, CfgA::BN>(bm.tri, m0, n0);
  }
  __device__ __forceinline__ void k_window(int64_t m0, int64_t& kbeg, int64_t& kend) const {
    tri_window<CfgA::BM>(bm.tri, m0, kbeg, kend);
  }
  __device__ __forceinline__ void apply4(int64_t m, int64_t n, f32x4 v) const {
    *reinterpret_cast<f32x4*>(out + n * ld + m) = v;
  }
  __device__ __forceinline__ float apply(int64_t, int64_t, float) const { return 0.0f; }
  __device__ __forceinline__ void colsum(int, int64_t, float) const {}
};

// The softmax's backward fused into the dP product: the product is computed
// transposed, dP^T = V dO^T [key][query], and each lane's four consecutive
// keys of one query become
//   dS[query][key] = P[query][key] (dP[query][key] - D[query]) * scale,
// rounded once to the storage dtype (8-byte loads of P, all issued before
// the tile's first store; 8-byte stores of dS). P is exactly 0 at masked keys, so dS is too; tiles wholly above the
// diagonal are skipped (kSkipLower) and never read by dQ or dK.
template <class S>
struct EpiSoftmaxGradTBatched {
  typename S::T* ds;
  const typename S::T* p;
  const float* drow;  // D [pairs][s]
  int64_t ld;         // s
  float scale;
  BatchMap bm;
  static constexpr bool kBatched = true;
  static constexpr bool kApply4 = true;
  static constexpr bool kFetch4 = true;
  static constexpr bool kColSum = false;
  struct Fetched {
    uint2 p;
    float d;
  };
  __device__ __forceinline__ void select(int z, Operand& P, Operand& Q) {
    const int64_t b = z / bm.inner, j = z % bm.inner;
    P.ptr += b * bm.p_b + j * bm.p_j;
    Q.ptr += b * bm.q_b + j * bm.q_j;
    const int64_t off = b * bm.o_b + j * bm.o_j;
    ds += off;
    p += off;
    drow += (int64_t)z * ld;
  }
  __device__ __forceinline__ bool skip(int64_t m0, int64_t n0) const {
    return tri_skip<CfgA::BM, CfgA::BN>(bm.tri, m0, n0);
  }
  __device__ __forceinline__ void k_window(int64_t m0, int64_t& kbeg, int64_t& kend) const {
    tri_window<CfgA::BM>(bm.tri, m0, kbeg, kend);
  }
  __device__ __forceinline__ Fetched fetch4(int64_t m, int64_t n) const {
    return Fetched{*reinterpret_cast<const uint2*>(p + n * ld + m), drow[n]};
  }
  __device__ __forceinline__ void apply4(int64_t m, int64_t n, f32x4 v, const Fetched& f) const {
    const uint2 w = f.p;
    const float dn = f.d;
    const float pv[4] = {S::to_f((typename S::T)(w.x & 0xffffu)), S::to_f((typename S::T)(w.x >> 16)),
                         S::to_f((typename S::T)(w.y & 0xffffu)), S::to_f((typename S::T)(w.y >> 16))};
    uint16_t r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = S::from_f(pv[i] * (v[i] - dn) * scale);
    *reinterpret_cast<uint2*>(ds + n * ld + m) =
        uint2{(uint32_t)r[0] | ((uint32_t)r[1] << 16), (uint32_t)r[2] | ((uint32_t)r[3] << 16)};
  }
  __device__ __forceinline__ float apply(int64_t, int64_t, float) const { return 0.0f; }
  __device__ __forceinline__ void colsum(int, int64_t, float) const {}
};

// C[M][N] = sum_k P[m][k] Q[k][n] for `batches` independent products (grid y).
template <class S, bool PK, bool QK, class Epi>
hipError_t gemm(int64_t M, int64_t N, int64_t K, const void* p, int64_t ldp, const void* q, int64_t ldq,
                const Epi& epi, int batches, hipStream_t st) {
  if (M == 0 || N == 0 || batches == 0) return hipSuccess;
  GemmShape sh{M, N, K, (int)cdiv(M, CfgA::BM), (int)cdiv(N, CfgA::BN), 1, std::max<int64_t>(K, 1)};
  hipLaunchKernelGGL((gemm_mfma_kernel<CfgA, S, PK, QK, false, Epi>), dim3(sh.tiles_m * sh.tiles_n, batches),
                     dim3(CfgA::THREADS), 0, st, sh, Operand{static_cast<const uint16_t*>(p), ldp},
                     Operand{static_cast<const uint16_t*>(q), ldq}, epi, RowSlices{});
  return hipGetLastError();
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Fused scale + causal mask + softmax, one wave per row of the fp32 scores
// [rows][s] (row r is query r % s of its (sequence, head) pair):
//   x_k = S[k] * scale for the visible keys k (k <= query when causal),
//   P[k] = exp(x_k - max) / sum_k' exp(x_k' - max), 0 for masked keys,
// rounded once to the storage dtype. Lane l holds keys 4 l + 256 c, c < CH,
// in registers (s <= 256 CH): the row is read from HBM once. The max and
// the sum are reduced per lane in key order, then across the wave in a
// fixed butterfly order.
template <class S, int CH>
__global__ __launch_bounds__(256) void softmax_fwd_kernel(const float* __restrict__ sc, typename S::T* __restrict__ P,
                                                          int64_t rows, int64_t s, float scale, int causal) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int64_t qi = row % s;
  const int64_t nv = causal ? qi + 1 : s;
  const float* x = sc + row * s;
  typename S::T* p = P + row * s;
  float v[CH][4];
  float m = -INFINITY;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t k = (int64_t)lane * 4 + 256 * c;
    float4 t = {0.f, 0.f, 0.f, 0.f};
    if (k < nv) t = *reinterpret_cast<const float4*>(x + k);
    v[c][0] = t.x * scale;
    v[c][1] = t.y * scale;
    v[c][2] = t.z * scale;
    v[c][3] = t.w * scale;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (k + i < nv) m = fmaxf(m, v[c][i]);
  }
  m = wave_max(m);
  float z = 0.0f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t k = (int64_t)lane * 4 + 256 * c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[c][i] = (k + i < nv) ? expf(v[c][i] - m) : 0.0f;
      z += v[c][i];
    }
  }
  z = wave_sum(z);
  const float rz = 1.0f / z;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t k = (int64_t)lane * 4 + 256 * c;
    if (k < s) {
      uint2 w;
      w.x = (uint32_t)S::from_f(v[c][0] * rz) | ((uint32_t)S::from_f(v[c][1] * rz) << 16);
      w.y = (uint32_t)S::from_f(v[c][2] * rz) | ((uint32_t)S::from_f(v[c][3] * rz) << 16);
      *reinterpret_cast<uint2*>(p + k) = w;
    }
  }
}

template <class S>
hipError_t softmax_fwd(const float* sc, typename S::T* P, int64_t rows, int64_t s, float scale, int causal,
                       hipStream_t st) {
  const dim3 grid((unsigned)cdiv(rows, 4)), block(256);
  if (s <= 256) hipLaunchKernelGGL((softmax_fwd_kernel<S, 1>), grid, block, 0, st, sc, P, rows, s, scale, causal);
  else if (s <= 512) hipLaunchKernelGGL((softmax_fwd_kernel<S, 2>), grid, block, 0, st, sc, P, rows, s, scale, causal);
  else if (s <= 1024) hipLaunchKernelGGL((softmax_fwd_kernel<S, 4>), grid, block, 0, st, sc, P, rows, s, scale, causal);
  else if (s <= 2048) hipLaunchKernelGGL((softmax_fwd_kernel<S, 8>), grid, block, 0, st, sc, P, rows, s, scale, causal);
  else hipLaunchKernelGGL((softmax_fwd_kernel<S, 16>), grid, block, 0, st, sc, P, rows, s, scale, causal);
  return hipGetLastError();
}

// Backward workspace: [D fp32 Z s][dS 16-bit Z s s][dO 16-bit T q]
// [column partials of dQKV fp32 [T/256][3q]][k-split partials of the
// projections' plain-store GEMMs (dO, dWo, dWqkv, dXp run one after the
// other and share the room)].
struct AttnBwdWs {
  size_t drow_off, ds_off, do_off, part_off, tail_off, tail_bytes, total;
  int part_blk;
};

AttnBwdWs bwd_layout(const AttnDims& a, int dtype) {
  AttnBwdWs w{};
  const size_t zss = (size_t)(a.Z * a.s * a.s);
  const int64_t T3 = 3 * a.q;
  w.drow_off = 0;
  w.ds_off = a256((size_t)(a.Z * a.s) * 4);
  w.do_off = w.ds_off + a256(zss * 2);
  w.part_off = w.do_off + a256((size_t)(a.T * a.q) * 2);
  w.part_blk = (int)cdiv(a.T, 256);
  w.tail_off = w.part_off + a256((size_t)w.part_blk * (size_t)T3 * 4);
  w.tail_bytes = std::max({planned_gemm_tail_bytes(dtype, a.T, a.q, a.h, true),
                           planned_gemm_tail_bytes(dtype, a.q, a.h, a.T, false),
                           planned_gemm_tail_bytes(dtype, a.h, T3, a.T, false),
                           planned_gemm_tail_bytes(dtype, a.T, a.h, T3, true)});
  w.total = w.tail_off + a256(w.tail_bytes);
  return w;
}

template <class S>
int attn_fwd_impl(const AttnDims& a, int dtype, int causal, const void* X, const void* Wqkv, const void* bqkv,
                  const void* Wo, void* QKV, void* P, void* O, void* Yp, void* ws, size_t ws_bytes, hipStream_t st) {
  using T = typename S::T;
  const int64_t T3 = 3 * a.q;
  const T* qkv = static_cast<const T*>(QKV);
  // QKV = X Wqkv + bqkv: P = X [T,h] k-contiguous, Q = Wqkv [h,3q] n-contiguous
  ATTN_HIP(planned_gemm(dtype, true, false, a.T, T3, a.h, X, a.h, Wqkv, T3, QKV, T3, bqkv, nullptr, 0, st));
  // S_bj [query][key] in fp32, computed as S^T = K_bj Q_bj^T [key][query] and stored transposed:
  // P = K block [s,d] k-contiguous, Q[k=d][n=query] = Q_bj[n][k] k-contiguous
  const BatchMap sc{(int)a.n, a.s * T3, a.d, a.s * T3, a.d, a.n * a.s * a.s, a.s * a.s, causal ? kSkipLower : kNone};
  ATTN_HIP((gemm<S, true, true>(a.s, a.s, a.d, qkv + a.q, T3, qkv, T3,
                                EpiStoreF32TBatched{static_cast<float*>(ws), a.s, sc}, (int)a.Z, st)));
  ATTN_HIP(softmax_fwd<S>(static_cast<const float*>(ws), static_cast<T*>(P), a.Z * a.s, a.s, a.scale, causal, st));
  // O_bj = P_bj V_bj: P_bj [s,s] k-contiguous, Q[k][n] = V[k][n] n-contiguous (pitch 3q)
  const BatchMap pv{(int)a.n, a.n * a.s * a.s, a.s * a.s, a.s * T3, a.d, a.s * a.q, a.d, causal ? kKeysUpTo : kNone};
  ATTN_HIP((gemm<S, true, false>(a.s, a.d, a.s, P, a.s, qkv + 2 * a.q, T3, EpiStoreBatched<S>{(T*)O, a.q, pv},
                                 (int)a.Z, st)));
  // Yp = O Wo: P = O [T,q] k-contiguous, Q = Wo [q,h] n-contiguous; the scores' room (free now)
  // takes the k-split partials if the plan has any and they fit
  ATTN_HIP(planned_gemm(dtype, true, false, a.T, a.h, a.q, O, a.q, Wo, a.h, Yp, a.h, nullptr,
                        static_cast<float*>(ws), ws_bytes, st));
  return TPMLP_OK;
}

template <class S>
int attn_bwd_impl(const AttnDims& a, int dtype, int causal, const void* dY, const void* X, const void* Wqkv,
                  const void* Wo, const void* QKV, const void* P, const void* O, void* dQKV, void* dXp, void* dWqkv,
                  void* dbqkv, void* dWo, void* ws, hipStream_t st) {
  using T = typename S::T;
  const int64_t T3 = 3 * a.q;
  const AttnBwdWs w = bwd_layout(a, dtype);
  char* wsb = static_cast<char*>(ws);
  float* drow = reinterpret_cast<float*>(wsb + w.drow_off);
  T* ds = reinterpret_cast<T*>(wsb + w.ds_off);
  T* dO = reinterpret_cast<T*>(wsb + w.do_off);
  float* part = reinterpret_cast<float*>(wsb + w.part_off);
  const T* qkv = static_cast<const T*>(QKV);
  T* dqkv = static_cast<T*>(dQKV);
  float* tail = reinterpret_cast<float*>(wsb + w.tail_off);
  // dO = dY Wo^T: Q[k=h][n=q] = Wo[n][k] k-contiguous
  ATTN_HIP(planned_gemm(dtype, true, true, a.T, a.q, a.h, dY, a.h, Wo, a.h, dO, a.q, nullptr, tail, w.tail_bytes, st));
  // dWo = O^T dY: P[m=q][k=T] = O[k][m], Q = dY [T,h]: both mn-contiguous
  ATTN_HIP(planned_gemm(dtype, false, false, a.q, a.h, a.T, O, a.q, dY, a.h, dWo, a.h, nullptr, tail, w.tail_bytes,
                        st));
  // dV_bj = P_bj^T dO_bj: P[m=key][k=query] = P_bj[k][m], Q = dO block: both mn-contiguous
  const BatchMap dv{(int)a.n, a.n * a.s * a.s, a.s * a.s, a.s * a.q, a.d, a.s * T3, a.d,
                    causal ? kQueriesFrom : kNone};
  ATTN_HIP((gemm<S, false, false>(a.s, a.d, a.s, P, a.s, dO, a.q, EpiStoreBatched<S>{dqkv + 2 * a.q, T3, dv},
                                  (int)a.Z, st)));
  // D = rowsum(dO * O) per (pair, query); then dP_bj = dO_bj V_bj^T, computed as dP^T = V_bj dO_bj^T
  // (P = V block k-contiguous, Q[k=d][n=query] = dO[n][k] k-contiguous), becomes dS in its epilogue
  hipLaunchKernelGGL(softmax_rowdot_kernel<S>, dim3((unsigned)cdiv(a.T * a.n, 256)), dim3(256), 0, st, dO,
                     static_cast<const T*>(O), drow, a.T, a.s, (int)a.n, (int)a.d, a.q);
  ATTN_HIP(hipGetLastError());
  const BatchMap dpm{(int)a.n, a.s * T3, a.d, a.s * a.q, a.d, a.n * a.s * a.s, a.s * a.s, causal ? kSkipLower : kNone};
  ATTN_HIP((gemm<S, true, true>(a.s, a.s, a.d, qkv + 2 * a.q, T3, dO, a.q,
                                EpiSoftmaxGradTBatched<S>{ds, static_cast<const T*>(P), drow, a.s, a.scale, dpm},
                                (int)a.Z, st)));
  // dQ_bj = dS_bj K_bj: P = dS [s,s] k-contiguous, Q[k=key][n=d] = K[k][n] n-contiguous
  const BatchMap dq{(int)a.n, a.n * a.s * a.s, a.s * a.s, a.s * T3, a.d, a.s * T3, a.d, causal ? kKeysUpTo : kNone};
  ATTN_HIP((gemm<S, true, false>(a.s, a.d, a.s, ds, a.s, qkv + a.q, T3, EpiStoreBatched<S>{dqkv, T3, dq},
                                 (int)a.Z, st)));
  // dK_bj = dS_bj^T Q_bj: P[m=key][k=query] = dS[k][m], Q[k=query][n=d] = Q[k][n]: both mn-contiguous
  BatchMap dk = dq;
  dk.tri = causal ? kQueriesFrom : kNone;
  ATTN_HIP((gemm<S, false, false>(a.s, a.d, a.s, ds, a.s, qkv, T3, EpiStoreBatched<S>{dqkv + a.q, T3, dk},
                                  (int)a.Z, st)));
  // dbqkv = column sums of dQKV
  hipLaunchKernelGGL(colsum_part_kernel<S>, dim3((unsigned)cdiv(T3, 256), (unsigned)w.part_blk), dim3(256), 0, st,
                     static_cast<const T*>(dQKV), a.T, T3, part);
  ATTN_HIP(hipGetLastError());
  hipLaunchKernelGGL(colsum_finish_kernel<S>, dim3((unsigned)cdiv(T3, 256)), dim3(256), 0, st, part, w.part_blk, T3,
                     static_cast<T*>(dbqkv));
  ATTN_HIP(hipGetLastError());
  // dWqkv = X^T dQKV: P[m=h][k=T] = X[k][m], Q = dQKV [T,3q]: both mn-contiguous
  ATTN_HIP(planned_gemm(dtype, false, false, a.h, T3, a.T, X, a.h, dQKV, T3, dWqkv, T3, nullptr, tail, w.tail_bytes,
                        st));
  // dXp = dQKV Wqkv^T: P = dQKV k-contiguous, Q[k=3q][n=h] = Wqkv[n][k] k-contiguous
  ATTN_HIP(planned_gemm(dtype, true, true, a.T, a.h, T3, dQKV, T3, Wqkv, T3, dXp, a.h, nullptr, tail, w.tail_bytes,
                        st));
  return TPMLP_OK;
}

}  // namespace
}  // namespace tpmlp

using namespace tpmlp;

extern "C" {

size_t tp_attn_fwd_workspace_bytes(const tpattn_shape* shape) {
  if (check_attn_shape(shape, false) != TPMLP_OK) return 0;
  const AttnDims a = dims(*shape);
  return a256((size_t)(a.Z * a.s * a.s) * 4);
}

size_t tp_attn_bwd_workspace_bytes(const tpattn_shape* shape) {
  if (check_attn_shape(shape, false) != TPMLP_OK) return 0;
  return bwd_layout(dims(*shape), shape->dtype).total;
}

int tp_attn_fwd(const tpattn_shape* shape, const void* X, const void* Wqkv, const void* bqkv, const void* Wo,
                void* QKV, void* P, void* O, void* Yp, void* ws, size_t ws_bytes, void* stream) {
  const int rc = check_attn_shape(shape, false);
  if (rc != TPMLP_OK) return rc;
  const AttnDims a = dims(*shape);
  const size_t e = 2, need = tp_attn_fwd_workspace_bytes(shape);
  const Span2 in[4] = {{X, (size_t)(a.T * a.h) * e}, {Wqkv, (size_t)(a.h * 3 * a.q) * e},
                       {bqkv, (size_t)(3 * a.q) * e}, {Wo, (size_t)(a.q * a.h) * e}};
  const Span2 out[5] = {{QKV, (size_t)(a.T * 3 * a.q) * e}, {P, (size_t)(a.Z * a.s * a.s) * e},
                        {O, (size_t)(a.T * a.q) * e}, {Yp, (size_t)(a.T * a.h) * e}, {ws, std::min(need, ws_bytes)}};
  const int bc = check_spans(in, 4, out, 5);
  if (bc != TPMLP_OK) return bc;
  if (ws_bytes < need) return TPMLP_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (shape->dtype == TPMLP_F16)
    return attn_fwd_impl<StoreF16>(a, shape->dtype, shape->causal, X, Wqkv, bqkv, Wo, QKV, P, O, Yp, ws, need, st);
  return attn_fwd_impl<StoreBF16>(a, shape->dtype, shape->causal, X, Wqkv, bqkv, Wo, QKV, P, O, Yp, ws, need, st);
}

int tp_attn_bwd(const tpattn_shape* shape, const void* dY, const void* X, const void* Wqkv, const void* Wo,
                const void* QKV, const void* P, const void* O, void* dQKV, void* dXp, void* dWqkv, void* dbqkv,
                void* dWo, void* ws, size_t ws_bytes, void* stream) {
  const int rc = check_attn_shape(shape, false);
  if (rc != TPMLP_OK) return rc;
  const AttnDims a = dims(*shape);
  const size_t e = 2, need = tp_attn_bwd_workspace_bytes(shape);
  const size_t Th = (size_t)(a.T * a.h) * e, T3 = (size_t)(a.T * 3 * a.q) * e, h3 = (size_t)(a.h * 3 * a.q) * e,
               qh = (size_t)(a.q * a.h) * e;
  const Span2 in[7] = {{dY, Th}, {X, Th}, {Wqkv, h3}, {Wo, qh}, {QKV, T3}, {P, (size_t)(a.Z * a.s * a.s) * e},
                       {O, (size_t)(a.T * a.q) * e}};
  const Span2 out[6] = {{dQKV, T3}, {dXp, Th}, {dWqkv, h3}, {dbqkv, (size_t)(3 * a.q) * e}, {dWo, qh},
                        {ws, std::min(need, ws_bytes)}};
  const int bc = check_spans(in, 7, out, 6);
  if (bc != TPMLP_OK) return bc;
  if (ws_bytes < need) return TPMLP_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (shape->dtype == TPMLP_F16)
    return attn_bwd_impl<StoreF16>(a, shape->dtype, shape->causal, dY, X, Wqkv, Wo, QKV, P, O, dQKV, dXp, dWqkv,
                                   dbqkv, dWo, ws, st);
  return attn_bwd_impl<StoreBF16>(a, shape->dtype, shape->causal, dY, X, Wqkv, Wo, QKV, P, O, dQKV, dXp, dWqkv,
                                  dbqkv, dWo, ws, st);
}

}  // extern "C"
