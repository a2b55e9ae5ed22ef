// Tile planning, workspace layouts, argument checks and GEMM launchers of the
// tensor-parallel MLP shard, shared by the translation units that hold its
// launch sequences (mlp_impl.hpp, one per storage type) and its C ABI
// (tp_mlp.hip).
//
// GEMMs that run on the direct-to-LDS engine read an operand fastest when it
// is k-contiguous. When the caller's workspace has room, the operands that
// are stored mn-contiguous (A_i and B_i in the forward; X, dY, H and dZ for
// the weight gradients) are first transposed into it by an HBM-bound kernel
// (TA, TB; TH, TdY, TX, TdZ), so all six GEMMs read k-contiguous tiles.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "tp_mlp.h"
#include "epilogues.hpp"
#include "gemm_dma.hpp"
#include "gemm_mfma.hpp"
#include "gemm_simt.hpp"
#include "transpose.hpp"

namespace tpmlp {

enum class Engine { Simt, Mfma128, Mfma256, Dma256, Dma320 };

using Cfg128 = MfmaTile<128, 128, 2, 2>;
using Cfg256 = MfmaTile<256, 256, 2, 4>;
using CfgD256 = DmaTile<256, 256, 2, 4, 64, 2>;
// 256 x 320 tiles (8 waves of 64 x 160): 10% fewer operand bytes per flop
// through L2 and LDS than 256 x 256; k-contiguous operands only (the
// mn-contiguous LDS swizzle assumes a power-of-two row of units).
using CfgD320 = DmaTile<256, 320, 4, 2, 64, 2>;

struct Plan {
  Engine eng;
  int bm, bn;
  int tiles_m, tiles_n;
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest operand (in elements) the direct-load engine addresses: byte
// offsets within one operand stay below 2^31.
constexpr int64_t kDmaMaxElems = (int64_t(1) << 30) - (int64_t(1) << 20);

// Row pitch of the transposed copies staged in the workspace: R + 256
// elements. A pitch that is a multiple of a large power of two (T = 16384
// tokens: 32 KB) sends the rows a GEMM tile reads together to few L2
// channels and sets; 512 bytes of padding per row spread them (measured on
// MI355X: 128 bytes do as much for the GEMMs but slow the transposes'
// stores by a sixth, 512 bytes do not).
constexpr int64_t kStagePad = 256;
inline int64_t staged_ld(int64_t R) { return R + kStagePad; }

// CUs of an MI355X: one wave of 256 x 256 tiles.
constexpr int kCUs = 256;

// The direct-load tiles on the 16x16x32 MFMA form (see gemm_dma.hpp), taken
// where the epilogue is tile-wise (not the fp32 read-modify-write) and the
// row pitches keep every load's offset below 2^31 (256 x 320 tiles only
// come with k-contiguous operands). With an mn-contiguous operand only in
// launches of at least one tile per CU: the form gains through the clock
// the chip holds under full load, and a launch that leaves CUs idle runs
// at a higher clock on either form, where the 16x16 one's doubled
// transposing reads cost more (measured on MI355X: 7B shard, 16 x 16
// tiles, dA 236 -> 230 us; 2.4B shard, 10 x 10 tiles split in two k-ranges,
// 126 -> 135 us).
using CfgD320x16 = DmaTile<256, 320, 4, 2, 64, 2, 1, true>;
using CfgD256x16 = DmaTile<256, 256, 2, 4, 64, 2, 1, true>;
template <class Epi>
inline constexpr bool kMf16Epi = !Epi::kDirectF32;
constexpr int64_t kMf16MaxLd = (int64_t(1) << 31) / (2 * CfgD320x16::BM);
inline std::atomic<bool> g_plan_mf16{true};
inline bool use_mf16(int64_t ldp, int64_t ldq, bool kc, int64_t) {
  return g_plan_mf16.load(std::memory_order_relaxed) && ldp < kMf16MaxLd && ldq < kMf16MaxLd && kc;
}

// Tile work of a launch counted in whole waves over the CUs (a last partial
// wave costs as much as a full one).
inline int64_t wave_cost(int64_t M, int64_t N, int bm, int bn) {
  return ceil_div(ceil_div(M, bm) * ceil_div(N, bn), kCUs) * bm * bn;
}

// A launch of fewer 256 x 256 tiles than this runs on 128 x 128 tiles
// (measured on MI355X: from about three quarters of a wave the direct-load
// engine's 256-wide tiles win, e.g. 1.3-1.6x on the 2560- and 4096-wide
// shards' GEMMs), unless it is a long reduction that the k-split below
// spreads over the chip.
constexpr int64_t kDmaMinTiles = 192;
// Reductions at least this long may split a sub-wave launch into k-ranges:
// up to four, or up to eight for reductions of kSubWaveLongK or more (the
// fp32 partials cost parts x tile bytes each way, which a long reduction's
// ranges amortise; measured on MI355X: eight ranges of K = 4096 GEMMs were
// slower than four, of K = 8192 ones faster).
constexpr int64_t kSubWaveSplitK = 2048;
constexpr int64_t kSubWaveLongK = 8192;
inline int subwave_max_parts(int64_t K) { return K >= kSubWaveLongK ? 8 : 4; }

// k-ranges per tile of a launch of `ntile` tiles that plan_tail splits as a
// sub-wave launch (1 if it does not).
inline int subwave_parts(int64_t ntile, int64_t K) {
  if (ntile > kCUs / 2 || K < kSubWaveSplitK) return 1;
  int parts = (int)std::min<int64_t>(subwave_max_parts(K), kCUs / ntile);
  while (parts > 1 && K < (int64_t)parts * 128) --parts;
  return parts;
}

// Cost of a k-split sub-wave launch: whole waves of its work items times the
// multiply-adds of one item, plus kPartialCost per fp32 partial element
// (written by the GEMM, read back by the finish). The weight is a fit to
// MI355X timings of such launches (e.g. 8192 x 640 x 2560: 256 x 320 tiles in
// four ranges, 50 us, against 256 x 256 tiles in two, 43 us; the tile work
// alone ranks them the other way).
constexpr int64_t kPartialCost = 7;
inline int64_t subwave_cost(int64_t M, int64_t N, int64_t K, int bm, int bn) {
  const int64_t ntile = ceil_div(M, bm) * ceil_div(N, bn);
  const int parts = subwave_parts(ntile, K);
  const int64_t partials = parts > 1 ? ntile * parts * bm * bn : 0;
  return ceil_div(ntile * parts, kCUs) * bm * bn * ceil_div(K, parts) + kPartialCost * partials;
}

// A launch of 16 .. kCUs / 2 tiles of 256 x 256 with a reduction of at least
// kSubWaveSplitK: plan_tail splits it into k-ranges.
inline bool subwave_split_candidate(int64_t M, int64_t N, int64_t K) {
  const int64_t t256 = ceil_div(M, 256) * ceil_div(N, 256);
  return t256 >= 16 && t256 <= kCUs / 2 && K >= kSubWaveSplitK;
}

// Tile choice for the 16-bit engines. Large tiles (256x256) once they give
// at least kDmaMinTiles of them (or at least 16 with a reduction of
// kSubWaveSplitK or more, which plan_tail splits into k-ranges), else
// 128x128. Large tiles use the direct-to-LDS engine unless P needs the GeLU
// applied on load (that engine has no register stage to apply it in) or an
// operand is too large for its 32-bit offsets; with both operands
// k-contiguous (kc) it takes 256x320 tiles unless they cost more whole
// waves. tp_mlp_debug_plan can force one engine where it applies (tests and
// tuning only).
inline std::atomic<int> g_plan_tile{TPMLP_PLAN_AUTO};
inline std::atomic<int> g_plan_cus{0};

inline Engine pick_engine(int64_t M, int64_t N, int64_t K, bool gelu_p, bool kc) {
  const bool dma_fits = !gelu_p && M * (K + kStagePad) <= kDmaMaxElems && N * (K + kStagePad) <= kDmaMaxElems;
  switch (g_plan_tile.load(std::memory_order_relaxed)) {
    case TPMLP_PLAN_REG128: return Engine::Mfma128;
    case TPMLP_PLAN_REG256: return Engine::Mfma256;
    case TPMLP_PLAN_DMA256: return dma_fits ? Engine::Dma256 : Engine::Mfma256;
    case TPMLP_PLAN_DMA320:
    case TPMLP_PLAN_DMA320_M32: return !dma_fits ? Engine::Mfma256 : kc ? Engine::Dma320 : Engine::Dma256;
    default: break;
  }
  const int64_t t256 = ceil_div(M, 256) * ceil_div(N, 256);
  const bool split_candidate = subwave_split_candidate(M, N, K);
  if (t256 < kDmaMinTiles && !split_candidate) return Engine::Mfma128;
  if (!dma_fits) return Engine::Mfma256;
  if (kc && split_candidate)  // the k-split's work items decide which tile fills the chip better
    return subwave_cost(M, N, K, CfgD320::BM, CfgD320::BN) < subwave_cost(M, N, K, CfgD256::BM, CfgD256::BN)
               ? Engine::Dma320
               : Engine::Dma256;
  if (kc && wave_cost(M, N, CfgD320::BM, CfgD320::BN) <= wave_cost(M, N, CfgD256::BM, CfgD256::BN))
    return Engine::Dma320;
  return Engine::Dma256;
}

// kc: both operands k-contiguous.
inline Plan plan_gemm(int dtype, int64_t M, int64_t N, int64_t K, bool gelu_p, bool kc) {
  Plan p;
  p.eng = dtype == TPMLP_F32 ? Engine::Simt : pick_engine(M, N, K, gelu_p, kc);
  switch (p.eng) {
    case Engine::Simt: p.bm = SimtTile::BM; p.bn = SimtTile::BN; break;
    case Engine::Mfma128: p.bm = Cfg128::BM; p.bn = Cfg128::BN; break;
    case Engine::Mfma256: p.bm = Cfg256::BM; p.bn = Cfg256::BN; break;
    case Engine::Dma256: p.bm = CfgD256::BM; p.bn = CfgD256::BN; break;
    case Engine::Dma320: p.bm = CfgD320::BM; p.bn = CfgD320::BN; break;
  }
  p.tiles_m = (int)ceil_div(M, p.bm);
  p.tiles_n = (int)ceil_div(N, p.bn);
  return p;
}

template <class Cfg, class S, bool PK, bool QK, bool GP, class Epi, bool SL = false>
void launch_mfma(const GemmShape& sh, const void* p, int64_t ldp, const void* q, int64_t ldq, const Epi& epi,
                 hipStream_t st, const RowSlices& xs = RowSlices{}) {
  const int nblk = sh.tiles_m * sh.tiles_n * sh.splits;
  hipLaunchKernelGGL((gemm_mfma_kernel<Cfg, S, PK, QK, GP, Epi, SL>), dim3(nblk), dim3(Cfg::THREADS), 0, st, sh,
                     Operand{static_cast<const uint16_t*>(p), ldp}, Operand{static_cast<const uint16_t*>(q), ldq},
                     epi, xs);
}

// Split of the last partial wave of a direct-load GEMM (see TailSplit): when
// fewer than half the CUs would get a tile in the last wave, those tiles are
// split into up to four k-ranges of at least 128. A launch of less than half
// a wave is split the same way (every tile, into up to subwave_max_parts
// ranges) if its reduction is at least kSubWaveSplitK long. Only plain-store
// epilogues.
// tp_mlp_debug_plan can replace the CU count of this plan (lets tests
// exercise tail splits at small sizes).
inline TailSplit plan_tail(const Plan& pl, int64_t K, bool allowed) {
  const int ntile = pl.tiles_m * pl.tiles_n;
  TailSplit t{ntile, 1, K, nullptr};
  const int forced = g_plan_cus.load(std::memory_order_relaxed);
  const int cus = forced > 0 ? forced : kCUs;
  const int r = ntile % cus;
  const bool dma = pl.eng == Engine::Dma256 || pl.eng == Engine::Dma320;
  if (!allowed || !dma || r == 0 || r > cus / 2) return t;
  if (ntile < cus && K < kSubWaveSplitK) return t;
  int parts = std::min(ntile < cus ? subwave_max_parts(K) : 4, cus / r);
  while (parts > 1 && K < (int64_t)parts * 128) --parts;
  if (parts < 2) return t;
  t.full = ntile - r;
  t.k_part = ceil_div(ceil_div(K, parts), 64) * 64;
  t.parts = (int)ceil_div(K, t.k_part);  // every range non-empty
  if (t.parts < 2) return TailSplit{ntile, 1, K, nullptr};
  return t;
}

inline size_t tail_bytes(const TailSplit& t, const Plan& pl) {
  return t.parts > 1 ? (size_t)(pl.tiles_m * pl.tiles_n - t.full) * t.parts * pl.bm * pl.bn * sizeof(float) : 0;
}

template <class Cfg, class S, bool PK, bool QK, class Epi, bool SL = false>
hipError_t launch_dma(const GemmShape& sh, const void* p, int64_t ldp, const void* q, int64_t ldq, const Epi& epi,
                      TailSplit tail, hipStream_t st, const RowSlices& xs = RowSlices{}) {
  const int ntile = sh.tiles_m * sh.tiles_n;
  const int nwork = tail.full + (ntile - tail.full) * tail.parts;
  // one workgroup per CU, looping over the work items
  const int nblk = std::min(nwork, kCUs * Cfg::OCC);
  // operand extents in elements: rows (KC) or k-rows (MC) times the pitch
  hipLaunchKernelGGL((gemm_dma_kernel<Cfg, S, PK, QK, Epi, SL>), dim3(nblk), dim3(Cfg::THREADS), 0, st, sh,
                     Operand{static_cast<const uint16_t*>(p), ldp}, (PK ? sh.M : sh.K) * ldp,
                     Operand{static_cast<const uint16_t*>(q), ldq}, (QK ? sh.N : sh.K) * ldq, epi, tail, nwork, xs,
                     PairGemm<Epi>{nullptr, nullptr, epi, 0});
  if constexpr (Epi::kTailSplit) {
    if (tail.parts > 1) {
      const int ntail = ntile - tail.full;
      const int64_t threads = (int64_t)ntail * Cfg::BM * (Cfg::BN / 8);
      hipLaunchKernelGGL((tail_finish_kernel<S, Cfg::GROUP, Cfg::BM, Cfg::BN>), dim3((unsigned)ceil_div(threads, 256)),
                         dim3(256), 0, st, tail.partial, tail.full, ntail, tail.parts, sh.tiles_m, sh.tiles_n, sh.M,
                         sh.N, epi.out, epi.ld);
    }
  }
  return hipGetLastError();
}

// C[M][N] = sum_k P[m][k] Q[k][n] through epilogue `epi`; PK / QK select the
// k-contiguous layout of P / Q, GP applies gelu to P as it is loaded. ldp /
// ldq: row pitch in elements, at least the contiguous extent (K for a
// k-contiguous operand, M or N otherwise; larger only for the padded staged
// copies, which the direct-load engines read). tail_ws: room for the partials of
// a k-split last wave and its size in bytes; the split is taken only if
// its partials (tail_bytes(plan_tail(...))) fit.
template <class S, bool PK, bool QK, bool GP, class Epi>
hipError_t run_gemm(int dtype, int64_t M, int64_t N, int64_t K, const void* p, int64_t ldp, const void* q,
                    int64_t ldq, const Epi& epi, hipStream_t st, float* tail_ws = nullptr, size_t tail_cap = 0) {
  if (M == 0 || N == 0) return hipSuccess;
  const Plan pl = plan_gemm(dtype, M, N, K, GP, PK && QK);
  GemmShape sh{M, N, K, pl.tiles_m, pl.tiles_n, 1, std::max<int64_t>(K, 1)};
  if constexpr (std::is_same_v<S, StoreF32>) {
    hipLaunchKernelGGL((gemm_simt_kernel<PK, QK, GP, Epi>), dim3(pl.tiles_m * pl.tiles_n), dim3(SimtTile::THREADS),
                       0, st, sh, OperandF32{static_cast<const float*>(p), ldp},
                       OperandF32{static_cast<const float*>(q), ldq}, epi);
  } else {
    switch (pl.eng) {
      case Engine::Dma256:
        if constexpr (!GP) {
          TailSplit tail = plan_tail(pl, K, Epi::kTailSplit && tail_ws != nullptr);
          if (tail_bytes(tail, pl) > tail_cap) tail = TailSplit{pl.tiles_m * pl.tiles_n, 1, K, nullptr};
          tail.partial = tail_ws;
          if constexpr (kMf16Epi<Epi> && PK && QK)
            if (use_mf16(ldp, ldq, true, (int64_t)pl.tiles_m * pl.tiles_n))
              return launch_dma<CfgD256x16, S, PK, QK>(sh, p, ldp, q, ldq, epi, tail, st);
          return launch_dma<CfgD256, S, PK, QK>(sh, p, ldp, q, ldq, epi, tail, st);
        }
        break;
      case Engine::Dma320:
        if constexpr (!GP && PK && QK) {
          TailSplit tail = plan_tail(pl, K, Epi::kTailSplit && tail_ws != nullptr);
          if (tail_bytes(tail, pl) > tail_cap) tail = TailSplit{pl.tiles_m * pl.tiles_n, 1, K, nullptr};
          tail.partial = tail_ws;
          if constexpr (kMf16Epi<Epi>)
            if (use_mf16(ldp, ldq, true, 0)) return launch_dma<CfgD320x16, S, PK, QK>(sh, p, ldp, q, ldq, epi, tail, st);
          return launch_dma<CfgD320, S, PK, QK>(sh, p, ldp, q, ldq, epi, tail, st);
        }
        break;
      case Engine::Mfma256: launch_mfma<Cfg256, S, PK, QK, GP>(sh, p, ldp, q, ldq, epi, st); break;
      default: launch_mfma<Cfg128, S, PK, QK, GP>(sh, p, ldp, q, ldq, epi, st); break;
    }
  }
  return hipGetLastError();
}

// Two GEMMs of one shape, pitches and layout (the weight gradients dB and
// dA of a shard with f = h), each alone a launch of at most half a wave of
// 256 x 256 tiles, which plan_tail would split into k-ranges with fp32
// partials and a finishing pass: launched as one, their tiles fill up to a
// wave side by side, each over the whole reduction. Where the planner puts
// such a GEMM on the direct-load engine's 256 x 256 tiles and two of them
// fit in one wave of the CUs (the CU count that tp_mlp_debug_plan may
// replace, as for plan_tail).
inline bool pair_fits(int dtype, int64_t M, int64_t N, int64_t K, bool kc) {
  if (dtype == TPMLP_F32 || M <= 0 || N <= 0 || K <= 0) return false;
  const Plan pl = plan_gemm(dtype, M, N, K, false, kc);
  const int forced = g_plan_cus.load(std::memory_order_relaxed);
  const int cus = forced > 0 ? forced : kCUs;
  return pl.eng == Engine::Dma256 && 2 * pl.tiles_m * pl.tiles_n <= cus;
}

// C1 = P1 Q1 through epi1 and C2 = P2 Q2 through epi2 in one launch, where
// pair_fits (the caller checks); 256 x 256 tiles on the 32x32 MFMA form.
template <class S, bool PK, bool QK, class Epi>
hipError_t run_gemm_pair(int64_t M, int64_t N, int64_t K, const void* p1, const void* q1, const Epi& epi1,
                         const void* p2, const void* q2, const Epi& epi2, int64_t ldp, int64_t ldq,
                         hipStream_t st) {
  if constexpr (std::is_same_v<S, StoreF32>) {
    return hipErrorInvalidValue;  // pair_fits is false for fp32
  } else {
    using Cfg = CfgD256;
    const int tm = (int)ceil_div(M, Cfg::BM), tn = (int)ceil_div(N, Cfg::BN), ntile = tm * tn;
    const GemmShape sh{M, N, K, tm, tn, 1, K};
    const int nwork = 2 * ntile;
    hipLaunchKernelGGL((gemm_dma_kernel<Cfg, S, PK, QK, Epi, false, true>), dim3(std::min(nwork, kCUs * Cfg::OCC)),
                       dim3(Cfg::THREADS), 0, st, sh, Operand{static_cast<const uint16_t*>(p1), ldp},
                       (PK ? M : K) * ldp, Operand{static_cast<const uint16_t*>(q1), ldq}, (QK ? N : K) * ldq, epi1,
                       TailSplit{ntile, 1, K, nullptr}, nwork, RowSlices{},
                       PairGemm<Epi>{static_cast<const uint16_t*>(p2), static_cast<const uint16_t*>(q2), epi2, ntile});
    return hipGetLastError();
  }
}

// run_gemm with P (k-contiguous, [M][K]) read from row slices xs (see
// RowSlices; xs.rows rows each). The direct-load engines take it when every
// slice holds whole tiles of their BM rows, so that no tile straddles two
// slices; otherwise the register-staged engines, which map each row to its
// slice. No k-split (the first GEMM of the forward, which has none).
template <class S, bool QK, class Epi>
hipError_t run_gemm_sliced(int dtype, int64_t M, int64_t N, int64_t K, const RowSlices& xs, int64_t ldp,
                           const void* q, int64_t ldq, const Epi& epi, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  Plan pl = plan_gemm(dtype, M, N, K, false, QK);
  if ((pl.eng == Engine::Dma256 || pl.eng == Engine::Dma320) && xs.rows % pl.bm != 0) {
    pl.eng = ceil_div(M, 256) * ceil_div(N, 256) >= kDmaMinTiles ? Engine::Mfma256 : Engine::Mfma128;
    pl.bm = pl.eng == Engine::Mfma256 ? Cfg256::BM : Cfg128::BM;
    pl.bn = pl.eng == Engine::Mfma256 ? Cfg256::BN : Cfg128::BN;
    pl.tiles_m = (int)ceil_div(M, pl.bm);
    pl.tiles_n = (int)ceil_div(N, pl.bn);
  }
  GemmShape sh{M, N, K, pl.tiles_m, pl.tiles_n, 1, std::max<int64_t>(K, 1)};
  const TailSplit none{pl.tiles_m * pl.tiles_n, 1, K, nullptr};
  if constexpr (std::is_same_v<S, StoreF32>) {
    return hipErrorInvalidValue;  // the fp32 path reads dense operands only
  } else {
    switch (pl.eng) {
      case Engine::Dma256:
        if constexpr (kMf16Epi<Epi> && QK)
          if (use_mf16(ldp, ldq, true, (int64_t)pl.tiles_m * pl.tiles_n))
            return launch_dma<CfgD256x16, S, true, QK, Epi, true>(sh, nullptr, ldp, q, ldq, epi, none, st, xs);
        return launch_dma<CfgD256, S, true, QK, Epi, true>(sh, nullptr, ldp, q, ldq, epi, none, st, xs);
      case Engine::Dma320:  // planned for k-contiguous Q only
        if constexpr (QK) {
          if constexpr (kMf16Epi<Epi>)
            if (use_mf16(ldp, ldq, true, 0))
              return launch_dma<CfgD320x16, S, true, QK, Epi, true>(sh, nullptr, ldp, q, ldq, epi, none, st, xs);
          return launch_dma<CfgD320, S, true, QK, Epi, true>(sh, nullptr, ldp, q, ldq, epi, none, st, xs);
        } else {
          return launch_dma<CfgD256, S, true, QK, Epi, true>(sh, nullptr, ldp, q, ldq, epi, none, st, xs);
        }
      case Engine::Mfma256: launch_mfma<Cfg256, S, true, QK, false, Epi, true>(sh, nullptr, ldp, q, ldq, epi, st, xs); break;
      default: launch_mfma<Cfg128, S, true, QK, false, Epi, true>(sh, nullptr, ldp, q, ldq, epi, st, xs); break;
    }
  }
  return hipGetLastError();
}

// Bytes of tail partials a plain-store GEMM of this shape uses (0 if none);
// kc: both operands k-contiguous.
inline size_t gemm_tail_bytes(int dtype, int64_t M, int64_t N, int64_t K, bool kc) {
  if (dtype == TPMLP_F32 || M == 0 || N == 0) return 0;
  const Plan pl = plan_gemm(dtype, M, N, K, false, kc);
  return tail_bytes(plan_tail(pl, K, true), pl);
}

inline size_t elt_size(int dtype) { return dtype == TPMLP_F32 ? 4 : 2; }

constexpr int64_t kMaxDim = int64_t(1) << 30;

inline int check_shape(const tpmlp_shape* s) {
  if (!s) return TPMLP_ERR_NULL;
  if (s->dtype != TPMLP_F32 && s->dtype != TPMLP_F16 && s->dtype != TPMLP_BF16) return TPMLP_ERR_DTYPE;
  const int64_t d[3] = {s->tokens, s->hidden, s->ffn_shard};
  const int64_t mult = s->dtype == TPMLP_F32 ? 4 : 8;
  for (int64_t v : d) {
    if (v < 0 || v > kMaxDim) return TPMLP_ERR_SHAPE;
  }
  // the smallest tiles (64) must give a grid that fits in 31 bits
  if (ceil_div(s->tokens, 64) * ceil_div(std::max(s->hidden, s->ffn_shard), 64) > INT32_MAX / 2 ||
      ceil_div(s->hidden, 64) * ceil_div(s->ffn_shard, 64) > INT32_MAX / 2)
    return TPMLP_ERR_SHAPE;
  for (int64_t v : d) {
    if (v % mult) return TPMLP_ERR_ALIGN;
  }
  if (s->layout & ~(TPMLP_LAYOUT_B_T | TPMLP_LAYOUT_WEIGHTS_STAGED)) return TPMLP_ERR_SHAPE;
  return TPMLP_OK;
}

// The second weight arrives as B_i^T [h][f] (and dB leaves as [h][f]).
inline bool b_t(const tpmlp_shape& s) { return (s.layout & TPMLP_LAYOUT_B_T) != 0; }
// The forward workspace already holds the weight copies (the caller's promise).
inline bool weights_staged(const tpmlp_shape& s) { return (s.layout & TPMLP_LAYOUT_WEIGHTS_STAGED) != 0; }

struct Span {
  const void* p;
  size_t bytes;
};

inline bool overlap(const Span& a, const Span& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Required pointers (non-empty tensors) must be non-null; every non-null
// pointer must be 16-byte aligned; outputs may not overlap anything else.
inline int check_buffers(const Span* in, int n_in, const bool* in_required, const Span* out, int n_out,
                  const bool* out_required) {
  for (int i = 0; i < n_in; ++i)
    if (in_required[i] && in[i].bytes && !in[i].p) return TPMLP_ERR_NULL;
  for (int i = 0; i < n_out; ++i)
    if (out_required[i] && out[i].bytes && !out[i].p) return TPMLP_ERR_NULL;
  for (int i = 0; i < n_in; ++i)
    if (((uintptr_t)in[i].p & 15u) != 0) return TPMLP_ERR_ALIGN;
  for (int i = 0; i < n_out; ++i)
    if (((uintptr_t)out[i].p & 15u) != 0) return TPMLP_ERR_ALIGN;
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlap(out[i], in[j])) return TPMLP_ERR_ALIAS;
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(out[i], out[j])) return TPMLP_ERR_ALIAS;
  }
  return TPMLP_OK;
}

// Records events[i] on st; a NULL array or a NULL entry records nothing (an
// event record between two kernels idles the GPU for a few microseconds, so
// callers that time one step ask for only the points they use).
inline int record(void* const* events, int i, hipStream_t st) {
  if (!events || !events[i]) return TPMLP_OK;
  return hipEventRecord(static_cast<hipEvent_t>(events[i]), st) == hipSuccess ? TPMLP_OK : TPMLP_ERR_HIP;
}

#define TPMLP_TRY(expr)              \
  do {                               \
    const int rc_ = (expr);          \
    if (rc_ != TPMLP_OK) return rc_; \
  } while (0)
#define TPMLP_HIP(expr)                                 \
  do {                                                  \
    if ((expr) != hipSuccess) return TPMLP_ERR_HIP;     \
  } while (0)

// Transpose a dense [R][C] 16-bit matrix into out [C][staged_ld(R)] (gelu
// applied on the way when GELU).
template <class S, bool GELU>
hipError_t run_transpose(const void* in, void* out, int64_t R, int64_t C, hipStream_t st) {
  if (R == 0 || C == 0) return hipSuccess;
  const int tiles_c = (int)ceil_div(C, kTrCols), tiles_r = (int)ceil_div(R, kTrWaveTile);
  hipLaunchKernelGGL((transpose16_kernel<S, GELU>), dim3(tiles_r * tiles_c), dim3(64 * kTrWaves), 0, st,
                     static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out), R, C, staged_ld(R), tiles_c);
  return hipGetLastError();
}

// Does staging k-contiguous copies of a GEMM's mn-contiguous operands pay
// off? For the weight gradients (both operands [rows][T]) only where the
// copies buy the 256 x 320 tiles for a launch of a wave or more: with both
// operands k-contiguous the planner picks them, and that tile reads
// k-contiguous operands only. Where they would take 256 x 256 tiles anyway,
// the direct-load engine reads the operands in place with transposing LDS
// reads, and on MI355X that cost less than the two copies (the 7B shard's
// 4096 x 4096 x 8192 weight gradient: 204 us in place against 233 us for
// the copies and the GEMM). Where the copies buy the 320-wide tiles they
// win or tie: at h=10240, 16384 x 10240 x 10240 with one such operand
// 2.57 ms in place against 2.39 ms for its copy and the GEMM, a 10240 x
// 10240 x 16384 weight gradient 2.61 against 2.63 ms. A k-split sub-wave
// launch is not staged either: its copies scale with the long reduction
// while its tiles do not (the 2.4B shard's weight gradients, 2560 x 2560 x
// 8192: 123 us in place against 133 us for the two copies and the
// 320-wide GEMM). A forward weight is copied on more occasions
// (stages_weight).
inline bool stages(int dtype, int64_t M, int64_t N, int64_t K) {
  if (dtype == TPMLP_F32 || M <= 0 || N <= 0 || K <= 0) return false;
  if (subwave_split_candidate(M, N, K)) return false;
  return pick_engine(M, N, K, false, true) == Engine::Dma320;
}

// A GEMM whose one mn-contiguous operand is a weight ([h][f] or [f][h], far
// smaller than the token-long operands): staged as stages() says, and also
// where it takes 256 x 256 tiles on the direct-load engine, since there the
// copy buys the 16x16 MFMA form, which reads k-contiguous operands only.
// Measured on MI355X, the 7B shard's forward (8192 x 4096 x 4096, fp16):
// the first GEMM 225 us plus a 10 us copy against 250 us in place, the
// second 212 plus 11 against 234 us.
inline bool stages_weight(int dtype, int64_t M, int64_t N, int64_t K) {
  if (stages(dtype, M, N, K)) return true;
  if (dtype == TPMLP_F32 || M <= 0 || N <= 0 || K <= 0 || subwave_split_candidate(M, N, K)) return false;
  return pick_engine(M, N, K, false, true) == Engine::Dma256 && staged_ld(K) < kMf16MaxLd;
}

inline size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// Forward workspace: [A_i^T [f][h + pad]] [B_i^T [h][f + pad]] (each only
// if its GEMM stages) [tail partials of the second GEMM].
struct FwdWs {
  size_t at_off, bt_off, tail_off, tail_bytes, total;
  bool at, bt;
};

inline FwdWs fwd_ws(const tpmlp_shape& s) {
  FwdWs w{};
  const size_t e = elt_size(s.dtype);
  const size_t at_b = (size_t)(s.ffn_shard * staged_ld(s.hidden)) * e, bt_b = (size_t)(s.hidden * staged_ld(s.ffn_shard)) * e;
  w.at = stages_weight(s.dtype, s.tokens, s.ffn_shard, s.hidden);
  // B_i^T given (b_t): already the k-contiguous operand of F2, nothing to stage
  w.bt = !b_t(s) && stages_weight(s.dtype, s.tokens, s.hidden, s.ffn_shard);
  w.at_off = 0;
  w.bt_off = w.at ? align256(at_b) : 0;
  w.tail_off = w.bt_off + (w.bt ? align256(bt_b) : 0);
  w.tail_bytes = gemm_tail_bytes(s.dtype, s.tokens, s.hidden, s.ffn_shard, w.bt || b_t(s));
  w.total = w.tail_off + align256(w.tail_bytes);
  return w;
}

// Backward workspace: [dZ (if kept here)] [db1 partials fp32 [tiles][f]]
// then, when the weight-gradient GEMMs stage: [H^T][dY^T] for dB and
// [X^T][dZ^T] for dA (each [rows][T + pad]); with B_i^T given, B_i
// [f][h + pad] for the dZ GEMM when it stages; then the tail partials of the
// plain-store GEMMs (dB, dA, dXp run one after another and share them).
struct BwdWs {
  size_t dz_off, dz_bytes, part_off, part_bytes, minimal;
  size_t ht_off, dyt_off, xt_off, dzt_off, bs_off, tail_off, tail_bytes, total;
  int part_tiles;
  bool stage_b2, stage_b3, stage_b1;
};

inline BwdWs bwd_ws(const tpmlp_shape& s, bool dz_in_ws) {
  BwdWs w{};
  const size_t e = elt_size(s.dtype);
  const Plan b1 = plan_gemm(s.dtype, s.tokens, s.ffn_shard, s.hidden, false, true);
  w.part_tiles = (s.tokens > 0 && s.ffn_shard > 0) ? b1.tiles_m : 0;
  w.dz_off = 0;
  w.dz_bytes = dz_in_ws ? (size_t)(s.tokens * s.ffn_shard) * e : 0;
  w.part_off = align256(w.dz_bytes);
  w.part_bytes = (size_t)w.part_tiles * (size_t)s.ffn_shard * sizeof(float);
  w.minimal = w.part_bytes ? w.part_off + w.part_bytes : w.dz_bytes;
  w.stage_b2 = stages(s.dtype, s.ffn_shard, s.hidden, s.tokens);
  w.stage_b3 = stages(s.dtype, s.hidden, s.ffn_shard, s.tokens);
  const size_t tf = align256((size_t)(staged_ld(s.tokens) * s.ffn_shard) * e),
               th = align256((size_t)(staged_ld(s.tokens) * s.hidden) * e);
  size_t at = align256(w.minimal);
  if (w.stage_b2) {
    w.ht_off = at;
    w.dyt_off = at + tf;
    at += tf + th;
  }
  if (w.stage_b3) {
    w.xt_off = at;
    w.dzt_off = at + th;
    at += th + tf;
  }
  w.stage_b1 = b_t(s) && stages_weight(s.dtype, s.tokens, s.ffn_shard, s.hidden);
  if (w.stage_b1) {
    w.bs_off = at;
    at += align256((size_t)(s.ffn_shard * staged_ld(s.hidden)) * e);
  }
  // dB is the same GEMM with its operands swapped when B_i^T is given
  const size_t tail = std::max({gemm_tail_bytes(s.dtype, s.ffn_shard, s.hidden, s.tokens, w.stage_b2),
                                 gemm_tail_bytes(s.dtype, s.hidden, s.ffn_shard, s.tokens, w.stage_b2),
                                 gemm_tail_bytes(s.dtype, s.hidden, s.ffn_shard, s.tokens, w.stage_b3),
                                 gemm_tail_bytes(s.dtype, s.tokens, s.hidden, s.ffn_shard, true)});
  w.tail_off = at;
  w.tail_bytes = tail;
  w.total = (w.stage_b2 || w.stage_b3 || w.stage_b1 || tail) ? at + align256(tail) : w.minimal;
  return w;
}

// Workspace front of the recomputing backward: [Z_i [T][f]] then, when the
// first GEMM stages, [A_i^T [f][h + pad]]; the backward's own workspace
// follows at `bytes`.
struct RcWs {
  size_t at_off, bytes;
  bool at;
};

inline RcWs rc_ws(const tpmlp_shape& s) {
  RcWs r{};
  const size_t e = elt_size(s.dtype);
  r.at = stages_weight(s.dtype, s.tokens, s.ffn_shard, s.hidden);
  r.at_off = align256((size_t)(s.tokens * s.ffn_shard) * e);
  r.bytes = r.at_off + (r.at ? align256((size_t)(s.ffn_shard * staged_ld(s.hidden)) * e) : 0);
  return r;
}

}  // namespace tpmlp
