// MFMA GEMM engine for gfx950: C[M][N] = sum_k P[m][k] Q[k][n], 16-bit
// operands, fp32 accumulation in v_mfma_f32_16x16x32_{f16,bf16}.
//
// Operand layouts. Each operand is either k-contiguous ("KC": P[m][k] at
// p[m*ld + k], Q[k][n] at q[n*ld + k]) or mn-contiguous ("MC": P[m][k] at
// p[k*ld + m], Q[k][n] at q[k*ld + n]). The six GEMMs of the MLP shard use
// all three combinations: forward (KC, MC), the dH and dXp GEMMs (KC, KC),
// the weight gradients (MC, MC).
//
// Staging. Tiles of BM x 64 (P) and BN x 64 (Q) go global -> VGPR -> LDS with
// 16-byte loads and stores, double-buffered in LDS (one barrier per 64-wide
// K step; the next step's global loads are in flight while the current
// step's MFMAs run). Each operand keeps its global layout in LDS:
//   KC tile: [rows][64 k], 128-byte rows of eight 16-byte chunks, chunk index
//            XOR-swizzled by the row so that 16 lanes reading 16 rows at the
//            same k hit distinct banks;
//   MC tile: [64 k][rows], rows of 32-byte chunks XOR-swizzled by k.
// MFMA fragments (lane l holds row l%16, eight consecutive k starting at
// 8*(l/16)) come from a KC tile with one ds_read_b128 and from an MC tile
// with two ds_read_b64_tr_b16 transposing reads, so neither layout needs a
// register transpose.
//
// Workgroup -> tile order. gfx950 places workgroup b on XCD b % 8, and each
// XCD has its own L2. Workgroup ids are renumbered so that each XCD receives
// a contiguous range of tiles, walked GROUP tile-rows at a time, so that the
// tiles that run together on one XCD share A row panels and B column panels.
#pragma once

#include <type_traits>

#include "numerics.hpp"

namespace tpmlp {

// A batched epilogue (static constexpr bool kBatched = true) serves a grid
// whose y index z selects one of several independent GEMMs of the same
// shape: its select(z, P, Q) moves the two operands and its own outputs to
// batch z's matrices before the tile is computed. It also bounds the work of
// a tile: skip(m0, n0) drops a tile whose outputs are never read, and
// k_window(m0, kbeg, kend) narrows its k-range to where the operands can be
// nonzero (both for the triangular structure of causal attention; the
// narrowed range must start on a multiple of 64).
template <class E, class = void>
struct EpiBatched : std::false_type {};
template <class E>
struct EpiBatched<E, std::void_t<decltype(E::kBatched)>> : std::integral_constant<bool, E::kBatched> {};

// An epilogue with kApply4 = true takes each lane's four accumulators of a
// 16x16 fragment at once: apply4(m, n, v) with v[r] = C[m + r][n], m a
// multiple of 4 (M must then be a multiple of 4).
template <class E, class = void>
struct EpiApply4 : std::false_type {};
template <class E>
struct EpiApply4<E, std::void_t<decltype(E::kApply4)>> : std::integral_constant<bool, E::kApply4> {};

// An apply4 epilogue that also reads an input at the output positions
// (kFetch4 = true) splits the read off: fetch4(m, n) returns what
// apply4(m, n, v, fetched) needs. The kernel issues every fetch of the tile
// before its k-loop (the reads do not depend on the product), and so before
// the first store, which the compiler could not move them above.
template <class E, class = void>
struct EpiFetch4 : std::false_type {};
template <class E>
struct EpiFetch4<E, std::void_t<decltype(E::kFetch4)>> : std::integral_constant<bool, E::kFetch4> {};
struct NoFetchEpi {
  struct Fetched {};
};
template <class E>
using FetchedOf = typename std::conditional_t<EpiFetch4<E>::value, E, NoFetchEpi>::Fetched;

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct MfmaTile {
  static constexpr int BM = BM_, BN = BN_, BK = 64;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static constexpr int LDS_P = BM * BK * 2, LDS_Q = BN * BK * 2;
  static constexpr int LDS_STAGE = LDS_P + LDS_Q;
  static constexpr int LDS_BYTES = 2 * LDS_STAGE;
  static constexpr int CH_P = BM * 8 / THREADS, CH_Q = BN * 8 / THREADS;  // 16-byte chunks per thread
  static constexpr int GROUP = 8;
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(CH_P * THREADS == BM * 8 && CH_Q * THREADS == BN * 8, "tile not divisible by threads");
  static_assert(BM >= 64 && BN >= 64, "MC swizzle needs at least four 32-byte chunks per row");
};

struct GemmShape {
  int64_t M, N, K;
  int tiles_m, tiles_n;
  int splits;      // K partitions (1 = no split)
  int64_t k_per;   // K elements per partition, a multiple of 64
};

struct Operand {
  const uint16_t* ptr;
  int64_t ld;  // elements between consecutive rows in memory
};

// A k-contiguous operand held as equal slices of rows in separate buffers
// (the token rows of X under sequence parallelism, one slice per rank):
// row r lives in slice r / rows, at row r % rows of it, every slice with the
// operand's row pitch. Passed by value to the kernels that read it.
constexpr int kMaxSlices = 16;
struct RowSlices {
  const uint16_t* p[kMaxSlices];
  int64_t rows;  // rows per slice
};

__device__ __forceinline__ int swz_kc(int r) { return (r ^ (r >> 3)) & 7; }

template <int R>
__device__ __forceinline__ int swz_mc(int k) {
  return ((k & 3) | (((k >> 3) & 1) << 2)) & (R / 16 - 1);
}

// Renumber workgroups for XCD locality, then walk GROUP tile-rows at a time.
template <int GROUP>
__device__ __forceinline__ void map_tile(int b, int nblk, int tiles_m, int tiles_n, int& split, int& tm, int& tn) {
  const int per = nblk >> 3, rem = nblk & 7, x = b & 7, i = b >> 3;
  b = (x < rem) ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
  const int ntile = tiles_m * tiles_n;
  split = b / ntile;
  b -= split * ntile;
  const int gid = b / (GROUP * tiles_n);
  const int first = gid * GROUP;
  const int gsz = min(tiles_m - first, GROUP);
  const int in = b - gid * GROUP * tiles_n;
  tm = first + in % gsz;
  tn = in / gsz;
}

// One 16-byte chunk of operand rows [mn0, mn0+R) x k-range [k0, k0+64) from
// global memory (zero outside [0, MN) x [k0, kend)).
template <bool KC, int R, int THREADS>
__device__ __forceinline__ u32x4 load_chunk(const Operand& op, int64_t mn0, int64_t MN, int64_t k0,
                                            int64_t kend, int q) {
  int64_t mn, k;
  if constexpr (KC) {
    mn = mn0 + (q >> 3);
    k = k0 + ((q & 7) << 3);
  } else {
    constexpr int CPR = R / 8;  // chunks per k-row
    k = k0 + q / CPR;
    mn = mn0 + (q % CPR) * 8;
  }
  u32x4 v = {0u, 0u, 0u, 0u};
  if (mn < MN && k < kend) {
    const uint16_t* p = KC ? op.ptr + mn * op.ld + k : op.ptr + k * op.ld + mn;
    v = *reinterpret_cast<const u32x4*>(p);
  }
  return v;
}

// load_chunk of a k-contiguous operand held as row slices (see RowSlices).
template <int R>
__device__ __forceinline__ u32x4 load_chunk_sliced(const RowSlices& xs, int64_t ld, int64_t mn0, int64_t MN,
                                                   int64_t k0, int64_t kend, int q) {
  const int64_t mn = mn0 + (q >> 3), k = k0 + ((q & 7) << 3);
  u32x4 v = {0u, 0u, 0u, 0u};
  if (mn < MN && k < kend) {
    const int64_t s = mn / xs.rows;
    v = *reinterpret_cast<const u32x4*>(xs.p[s] + (mn - s * xs.rows) * ld + k);
  }
  return v;
}

template <bool KC, int R>
__device__ __forceinline__ int lds_chunk_offset(int q) {
  if constexpr (KC) {
    const int r = q >> 3, kc = q & 7;
    return r * 128 + ((kc ^ swz_kc(r)) << 4);
  } else {
    constexpr int CPR = R / 8;
    const int kr = q / CPR, c8 = q % CPR;
    return kr * (R * 2) + ((((c8 >> 1) ^ swz_mc<R>(kr))) << 5) + ((c8 & 1) << 4);
  }
}

// MFMA fragment of 16 rows starting at `row0` (multiple of 16) for k-step
// ks (32 wide) of the 64-wide LDS tile.
template <bool KC, int R>
__device__ __forceinline__ u32x4 read_frag(const char* tile, int row0, int ks, int lane) {
  if constexpr (KC) {
    const int r = row0 + (lane & 15);
    const int kc = ks * 4 + (lane >> 4);
    return *reinterpret_cast<const u32x4*>(tile + r * 128 + ((kc ^ swz_kc(r)) << 4));
  } else {
    const int g = lane >> 4, j = lane & 15;
    u32x4 out;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int kr = ks * 32 + g * 8 + hh * 4 + (j >> 2);
      const int off = kr * (R * 2) + ((((row0 >> 4) ^ swz_mc<R>(kr))) << 5) + ((j & 3) << 3);
      typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
      const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off));
      const u32x2 w = __builtin_bit_cast(u32x2, v);
      out[2 * hh] = w[0];
      out[2 * hh + 1] = w[1];
    }
    return out;
  }
}

// SLICED_P: P (k-contiguous) is read from the row slices xs instead of P.ptr.
template <class Cfg, class S, bool P_KC, bool Q_KC, bool GELU_P, class Epi, bool SLICED_P = false>
__global__ __launch_bounds__(Cfg::THREADS) void gemm_mfma_kernel(GemmShape sh, Operand P, Operand Q, Epi epi,
                                                                 RowSlices xs) {
  static_assert(!SLICED_P || P_KC, "row slices of a k-contiguous P only");
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, THREADS = Cfg::THREADS;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  int split, tm, tn;
  map_tile<Cfg::GROUP>(blockIdx.x, gridDim.x, sh.tiles_m, sh.tiles_n, split, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  int64_t kbeg = (int64_t)split * sh.k_per;
  int64_t kend = min(sh.K, kbeg + sh.k_per);
  if constexpr (EpiBatched<Epi>::value) {
    epi.select((int)blockIdx.y, P, Q);
    if (epi.skip(m0, n0)) return;
    epi.k_window(m0, kbeg, kend);
  }
  const int nk = kend > kbeg ? (int)((kend - kbeg + BK - 1) / BK) : 0;
  // An epilogue's reads of its own input do not depend on the product: they
  // are issued here, ahead of the k-loop, and land while it runs.
  FetchedOf<Epi> fe[Cfg::FM][Cfg::FN];
  if constexpr (EpiFetch4<Epi>::value) {
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j) {
        const int64_t n = n0 + wn * Cfg::WTN + j * 16 + (lane & 15);
        const int64_t m = m0 + wm * Cfg::WTM + i * 16 + (lane >> 4) * 4;
        if (m < sh.M && n < sh.N) fe[i][j] = epi.fetch4(m, n);
      }
  }

  f32x4 acc[Cfg::FM][Cfg::FN];
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 rp[Cfg::CH_P], rq[Cfg::CH_Q];
  auto load_stage = [&](int64_t k0) {
#pragma unroll
    for (int c = 0; c < Cfg::CH_P; ++c)
      if constexpr (SLICED_P)
        rp[c] = load_chunk_sliced<BM>(xs, P.ld, m0, sh.M, k0, kend, tid + c * THREADS);
      else
        rp[c] = load_chunk<P_KC, BM, THREADS>(P, m0, sh.M, k0, kend, tid + c * THREADS);
#pragma unroll
    for (int c = 0; c < Cfg::CH_Q; ++c)
      rq[c] = load_chunk<Q_KC, BN, THREADS>(Q, n0, sh.N, k0, kend, tid + c * THREADS);
  };
  auto store_stage = [&](int buf) {
    char* sp = smem + buf * Cfg::LDS_STAGE;
    char* sq = sp + Cfg::LDS_P;
#pragma unroll
    for (int c = 0; c < Cfg::CH_P; ++c) {
      u32x4 v = rp[c];
      if constexpr (GELU_P) v = gelu_chunk<S>(v);
      *reinterpret_cast<u32x4*>(sp + lds_chunk_offset<P_KC, BM>(tid + c * THREADS)) = v;
    }
#pragma unroll
    for (int c = 0; c < Cfg::CH_Q; ++c)
      *reinterpret_cast<u32x4*>(sq + lds_chunk_offset<Q_KC, BN>(tid + c * THREADS)) = rq[c];
  };

  if (nk > 0) {
    load_stage(kbeg);
    store_stage(0);
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
      const int cur = t & 1;
      if (t + 1 < nk) load_stage(kbeg + (int64_t)(t + 1) * BK);
      const char* sp = smem + cur * Cfg::LDS_STAGE;
      const char* sq = sp + Cfg::LDS_P;
#pragma unroll
      for (int ks = 0; ks < BK / 32; ++ks) {
        u32x4 fp[Cfg::FM], fq[Cfg::FN];
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i) fp[i] = read_frag<P_KC, BM>(sp, wm * Cfg::WTM + i * 16, ks, lane);
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) fq[j] = read_frag<Q_KC, BN>(sq, wn * Cfg::WTN + j * 16, ks, lane);
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
          for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = S::mfma16x16x32(fp[i], fq[j], acc[i][j]);
      }
      if (t + 1 < nk) store_stage(cur ^ 1);
      __syncthreads();
    }
  }

  // Epilogue. Lane l holds C[4*(l/16) + r][l % 16] of each 16x16 fragment.
  float cs[Cfg::FN];
#pragma unroll
  for (int j = 0; j < Cfg::FN; ++j) cs[j] = 0.0f;
  if constexpr (EpiFetch4<Epi>::value) {
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j) {
        const int64_t n = n0 + wn * Cfg::WTN + j * 16 + (lane & 15);
        const int64_t m = m0 + wm * Cfg::WTM + i * 16 + (lane >> 4) * 4;
        if (m < sh.M && n < sh.N) epi.apply4(m, n, acc[i][j], fe[i][j]);
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i) {
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int64_t n = n0 + wn * Cfg::WTN + j * 16 + (lane & 15);
      if constexpr (EpiApply4<Epi>::value && !EpiFetch4<Epi>::value) {
        const int64_t m = m0 + wm * Cfg::WTM + i * 16 + (lane >> 4) * 4;
        if (m < sh.M && n < sh.N) epi.apply4(m, n, acc[i][j]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t m = m0 + wm * Cfg::WTM + i * 16 + (lane >> 4) * 4 + r;
          if (m < sh.M && n < sh.N) cs[j] += epi.apply(m, n, acc[i][j][r]);
        }
      }
    }
  }
  if constexpr (Epi::kColSum) {
    // Column sums of this tile, in a fixed order: lanes, then waves.
    float* red = reinterpret_cast<float*>(smem);  // [WAVES_M][BN]; pipeline buffers are free now
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      cs[j] += __shfl_xor(cs[j], 16);
      cs[j] += __shfl_xor(cs[j], 32);
    }
    if (lane < 16) {
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j) red[wm * BN + wn * Cfg::WTN + j * 16 + lane] = cs[j];
    }
    __syncthreads();
    for (int c = tid; c < BN; c += THREADS) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < Cfg::WAVES_M; ++w) s += red[w * BN + c];
      if (n0 + c < sh.N) epi.colsum(tm, n0 + c, s);
    }
  }
}

}  // namespace tpmlp
