// C ABI of the tensor-parallel MLP shard (declared in include/tp_mlp.h):
// argument validation, tile planning and the launch sequences of the forward
// (F1: X A_i with fused bias + GeLU, F2: H_i B_i) and backward (B1: dY B_i^T
// with fused gelu' and db1 column partials, B5: db1 finish, B2: H_i^T dY,
// B3: X^T dZ_i, B4: dZ_i A_i^T).
//
// GEMMs that run on the direct-to-LDS engine read an operand fastest when it
// is k-contiguous. When the caller's workspace has room, the operands that
// are stored mn-contiguous (A_i and B_i in the forward; X, dY, H and dZ for
// the weight gradients) are first transposed into it by an HBM-bound kernel
// (TA, TB; TH, TdY, TX, TdZ), so all six GEMMs read k-contiguous tiles.
//
// tp_mlp_reduce_partials sums the row-parallel partials of P ranks held on
// this device (plus b2), over all rows or one rank's slice of rows.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "tp_mlp.h"
#include "colsum.hpp"
#include "epilogues.hpp"
#include "gemm_dma.hpp"
#include "gemm_mfma.hpp"
#include "gemm_simt.hpp"
#include "reduce.hpp"
#include "shard_gemm.hpp"
#include "transpose.hpp"

namespace tpmlp {
namespace {

// Device scratch of tp_mlp_bwd_static (the callers that cannot allocate):
// the fp32 column partials of dZ for db1. One copy per GPU, at its own
// address; host code uses the address hipGetSymbolAddress returns for the
// current device, never the array's name (a host-side stand-in).
static __device__ __align__(256) unsigned char scratch[TPMLP_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and cached.
int static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TPMLP_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TPMLP_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TPMLP_OK;
}

// Sum of the per-tile fp32 column partials [tiles_m][f], in a fixed order:
// a block of 256 threads covers 32 columns; thread (g, c) adds the tiles
// t = g, g + 8, g + 16, ... of column c in increasing t, then the 8 groups
// are added in group order. With ACC the sum is added to an fp32 main
// gradient (beta = 1); otherwise it is rounded once. Both forms add in the
// same order, so rounding the accumulated form (from zero) gives the other.
template <class S, bool ACC>
__global__ __launch_bounds__(256) void db1_finish_kernel(const float* partial, int tiles_m, int64_t f, void* db1) {
  __shared__ float red[8][32];
  const int c = threadIdx.x & 31, g = threadIdx.x >> 5;
  const int64_t n = (int64_t)blockIdx.x * 32 + c;
  float s = 0.0f;
  if (n < f)
    for (int t = g; t < tiles_m; t += 8) s += partial[(int64_t)t * f + n];
  red[g][c] = s;
  __syncthreads();
  if (g == 0 && n < f) {
    float v = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) v += red[k][c];
    if constexpr (ACC) static_cast<float*>(db1)[n] += v;
    else static_cast<typename S::T*>(db1)[n] = S::from_f(v);
  }
}

// Column sums of an fp32 [rows][cols] matrix, one thread per column, rows in
// order (the fp32 storage type's db2; its workloads are small).
template <bool ACC>
__global__ __launch_bounds__(256) void colsum_f32_kernel(const float* m, int64_t rows, int64_t cols, float* out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  float s = 0.0f;
  for (int64_t r = 0; r < rows; ++r) s += m[r * cols + c];
  if constexpr (ACC) out[c] += s;
  else out[c] = s;
}

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

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

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
int64_t staged_ld(int64_t R) { return R + kStagePad; }

// CUs of an MI355X: one wave of 256 x 256 tiles.
constexpr int kCUs = 256;

// Tile work of a launch counted in whole waves over the CUs (a last partial
// wave costs as much as a full one).
int64_t wave_cost(int64_t M, int64_t N, int bm, int bn) {
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
int subwave_max_parts(int64_t K) { return K >= kSubWaveLongK ? 8 : 4; }

// k-ranges per tile of a launch of `ntile` tiles that plan_tail splits as a
// sub-wave launch (1 if it does not).
int subwave_parts(int64_t ntile, int64_t K) {
  if (ntile > kCUs / 2 || K < kSubWaveSplitK) return 1;
  int parts = (int)std::min<int64_t>(subwave_max_parts(K), kCUs / ntile);
  while (parts > 1 && K < (int64_t)parts * 128) --parts;
  return parts;
}

// Cost of a k-split sub-wave launch in whole waves of its work items times
// the work of one item.
int64_t subwave_cost(int64_t M, int64_t N, int64_t K, int bm, int bn) {
  const int64_t ntile = ceil_div(M, bm) * ceil_div(N, bn);
  const int parts = subwave_parts(ntile, K);
  return ceil_div(ntile * parts, kCUs) * bm * bn * ceil_div(K, parts);
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
std::atomic<int> g_plan_tile{TPMLP_PLAN_AUTO};
std::atomic<int> g_plan_cus{0};

Engine pick_engine(int64_t M, int64_t N, int64_t K, bool gelu_p, bool kc) {
  const bool dma_fits = !gelu_p && M * (K + kStagePad) <= kDmaMaxElems && N * (K + kStagePad) <= kDmaMaxElems;
  switch (g_plan_tile.load(std::memory_order_relaxed)) {
    case TPMLP_PLAN_REG128: return Engine::Mfma128;
    case TPMLP_PLAN_REG256: return Engine::Mfma256;
    case TPMLP_PLAN_DMA256: return dma_fits ? Engine::Dma256 : Engine::Mfma256;
    case TPMLP_PLAN_DMA320: return !dma_fits ? Engine::Mfma256 : kc ? Engine::Dma320 : Engine::Dma256;
    default: break;
  }
  const int64_t t256 = ceil_div(M, 256) * ceil_div(N, 256);
  const bool split_candidate = t256 >= 16 && t256 <= kCUs / 2 && K >= kSubWaveSplitK;
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
Plan plan_gemm(int dtype, int64_t M, int64_t N, int64_t K, bool gelu_p, bool kc) {
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

template <class Cfg, class S, bool PK, bool QK, bool GP, class Epi>
void launch_mfma(const GemmShape& sh, const void* p, int64_t ldp, const void* q, int64_t ldq, const Epi& epi,
                 hipStream_t st) {
  const int nblk = sh.tiles_m * sh.tiles_n * sh.splits;
  hipLaunchKernelGGL((gemm_mfma_kernel<Cfg, S, PK, QK, GP, Epi>), dim3(nblk), dim3(Cfg::THREADS), 0, st, sh,
                     Operand{static_cast<const uint16_t*>(p), ldp}, Operand{static_cast<const uint16_t*>(q), ldq},
                     epi);
}

// Split of the last partial wave of a direct-load GEMM (see TailSplit): when
// fewer than half the CUs would get a tile in the last wave, those tiles are
// split into up to four k-ranges of at least 128. A launch of less than half
// a wave is split the same way (every tile, into up to subwave_max_parts
// ranges) if its reduction is at least kSubWaveSplitK long. Only plain-store
// epilogues.
// tp_mlp_debug_plan can replace the CU count of this plan (lets tests
// exercise tail splits at small sizes).
TailSplit plan_tail(const Plan& pl, int64_t K, bool allowed) {
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

size_t tail_bytes(const TailSplit& t, const Plan& pl) {
  return t.parts > 1 ? (size_t)(pl.tiles_m * pl.tiles_n - t.full) * t.parts * pl.bm * pl.bn * sizeof(float) : 0;
}

template <class Cfg, class S, bool PK, bool QK, class Epi>
hipError_t launch_dma(const GemmShape& sh, const void* p, int64_t ldp, const void* q, int64_t ldq, const Epi& epi,
                      TailSplit tail, hipStream_t st) {
  const int ntile = sh.tiles_m * sh.tiles_n;
  const int nwork = tail.full + (ntile - tail.full) * tail.parts;
  // one workgroup per CU, looping over the work items
  const int nblk = std::min(nwork, kCUs * Cfg::OCC);
  // operand extents in elements: rows (KC) or k-rows (MC) times the pitch
  hipLaunchKernelGGL((gemm_dma_kernel<Cfg, S, PK, QK, Epi>), dim3(nblk), dim3(Cfg::THREADS), 0, st, sh,
                     Operand{static_cast<const uint16_t*>(p), ldp}, (PK ? sh.M : sh.K) * ldp,
                     Operand{static_cast<const uint16_t*>(q), ldq}, (QK ? sh.N : sh.K) * ldq, epi, tail, nwork);
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
          return launch_dma<CfgD256, S, PK, QK>(sh, p, ldp, q, ldq, epi, tail, st);
        }
        break;
      case Engine::Dma320:
        if constexpr (!GP && PK && QK) {
          TailSplit tail = plan_tail(pl, K, Epi::kTailSplit && tail_ws != nullptr);
          if (tail_bytes(tail, pl) > tail_cap) tail = TailSplit{pl.tiles_m * pl.tiles_n, 1, K, nullptr};
          tail.partial = tail_ws;
          return launch_dma<CfgD320, S, PK, QK>(sh, p, ldp, q, ldq, epi, tail, st);
        }
        break;
      case Engine::Mfma256: launch_mfma<Cfg256, S, PK, QK, GP>(sh, p, ldp, q, ldq, epi, st); break;
      default: launch_mfma<Cfg128, S, PK, QK, GP>(sh, p, ldp, q, ldq, epi, st); break;
    }
  }
  return hipGetLastError();
}

// Bytes of tail partials a plain-store GEMM of this shape uses (0 if none);
// kc: both operands k-contiguous.
size_t gemm_tail_bytes(int dtype, int64_t M, int64_t N, int64_t K, bool kc) {
  if (dtype == TPMLP_F32 || M == 0 || N == 0) return 0;
  const Plan pl = plan_gemm(dtype, M, N, K, false, kc);
  return tail_bytes(plan_tail(pl, K, true), pl);
}

size_t elt_size(int dtype) { return dtype == TPMLP_F32 ? 4 : 2; }

constexpr int64_t kMaxDim = int64_t(1) << 30;

int check_shape(const tpmlp_shape* s) {
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
  if (s->layout & ~TPMLP_LAYOUT_B_T) return TPMLP_ERR_SHAPE;
  return TPMLP_OK;
}

// The second weight arrives as B_i^T [h][f] (and dB leaves as [h][f]).
bool b_t(const tpmlp_shape& s) { return (s.layout & TPMLP_LAYOUT_B_T) != 0; }

struct Span {
  const void* p;
  size_t bytes;
};

bool overlap(const Span& a, const Span& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Required pointers (non-empty tensors) must be non-null; every non-null
// pointer must be 16-byte aligned; outputs may not overlap anything else.
int check_buffers(const Span* in, int n_in, const bool* in_required, const Span* out, int n_out,
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

int record(void* const* events, int i, hipStream_t st) {
  if (!events) return TPMLP_OK;
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

// Does a GEMM of this shape run on the direct-to-LDS engine once all its
// operands are k-contiguous? (Then staging transposed copies pays off.)
bool stages(int dtype, int64_t M, int64_t N, int64_t K) {
  if (dtype == TPMLP_F32 || M <= 0 || N <= 0 || K <= 0) return false;
  const Engine e = pick_engine(M, N, K, false, true);
  return e == Engine::Dma256 || e == Engine::Dma320;
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// Forward workspace: [A_i^T [f][h + pad]] [B_i^T [h][f + pad]] (each only
// if its GEMM stages) [tail partials of the second GEMM].
struct FwdWs {
  size_t at_off, bt_off, tail_off, tail_bytes, total;
  bool at, bt;
};

FwdWs fwd_ws(const tpmlp_shape& s) {
  FwdWs w{};
  const size_t e = elt_size(s.dtype);
  const size_t at_b = (size_t)(s.ffn_shard * staged_ld(s.hidden)) * e, bt_b = (size_t)(s.hidden * staged_ld(s.ffn_shard)) * e;
  w.at = stages(s.dtype, s.tokens, s.ffn_shard, s.hidden);
  // B_i^T given (b_t): already the k-contiguous operand of F2, nothing to stage
  w.bt = !b_t(s) && stages(s.dtype, s.tokens, s.hidden, s.ffn_shard);
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

BwdWs bwd_ws(const tpmlp_shape& s, bool dz_in_ws) {
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
  w.stage_b1 = b_t(s) && stages(s.dtype, s.tokens, s.ffn_shard, s.hidden);
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

RcWs rc_ws(const tpmlp_shape& s) {
  RcWs r{};
  const size_t e = elt_size(s.dtype);
  r.at = stages(s.dtype, s.tokens, s.ffn_shard, s.hidden);
  r.at_off = align256((size_t)(s.tokens * s.ffn_shard) * e);
  r.bytes = r.at_off + (r.at ? align256((size_t)(s.ffn_shard * staged_ld(s.hidden)) * e) : 0);
  return r;
}

// Z = X A_i + b1 into `Z` (H not kept), the forward's first step; events 0-2
// bracket TA and F1.
template <class S>
int recompute_z(const tpmlp_shape& s, const void* X, const void* A, const void* b1, void* Z, const RcWs& r,
                char* wsb, hipStream_t st, void* const* ev) {
  using T = typename S::T;
  const int64_t Tn = s.tokens, h = s.hidden, f = s.ffn_shard;
  TPMLP_TRY(record(ev, 0, st));
  if (r.at) {
    TPMLP_HIP((run_transpose<S, false>(A, wsb + r.at_off, h, f, st)));
    TPMLP_TRY(record(ev, 1, st));
    TPMLP_HIP((run_gemm<S, true, true, false>(s.dtype, Tn, f, h, X, h, wsb + r.at_off, staged_ld(h),
                                              EpiBiasGelu<S>{(const T*)b1, (T*)Z, nullptr, f}, st)));
  } else {
    TPMLP_TRY(record(ev, 1, st));
    TPMLP_HIP((run_gemm<S, true, false, false>(s.dtype, Tn, f, h, X, h, A, f,
                                               EpiBiasGelu<S>{(const T*)b1, (T*)Z, nullptr, f}, st)));
  }
  return TPMLP_OK;
}

template <class S>
int fwd_impl(const tpmlp_shape& s, const void* X, const void* A, const void* b1, const void* B, void* Z, void* H,
             void* Yp, void* ws, size_t ws_bytes, hipStream_t st, void* const* ev) {
  using T = typename S::T;
  const int64_t Tn = s.tokens, h = s.hidden, f = s.ffn_shard;
  const FwdWs w = fwd_ws(s);
  const bool room = ws && ws_bytes >= w.total;
  char* wsb = static_cast<char*>(ws);
  TPMLP_TRY(record(ev, 0, st));
  // TA + F1: Z = X A_i + b1 (and H = gelu(Z)); P = X [T,h] k-contiguous,
  // Q = A_i [h,f] (n-contiguous), or its transpose A_i^T [f,h] (k-contiguous)
  if (room && w.at) {
    TPMLP_HIP((run_transpose<S, false>(A, wsb + w.at_off, h, f, st)));
    TPMLP_TRY(record(ev, 1, st));
    TPMLP_HIP((run_gemm<S, true, true, false>(s.dtype, Tn, f, h, X, h, wsb + w.at_off, staged_ld(h),
                                              EpiBiasGelu<S>{(const T*)b1, (T*)Z, (T*)H, f}, st)));
  } else {
    TPMLP_TRY(record(ev, 1, st));
    TPMLP_HIP((run_gemm<S, true, false, false>(s.dtype, Tn, f, h, X, h, A, f,
                                               EpiBiasGelu<S>{(const T*)b1, (T*)Z, (T*)H, f}, st)));
  }
  TPMLP_TRY(record(ev, 2, st));
  // TB + F2: Yp = H B_i (gelu(Z) on load when H is not kept); P [T,f]
  // k-contiguous, Q = B_i [f,h] (n-contiguous) or B_i^T [h,f] (k-contiguous)
  if (b_t(s)) {
    // B given as B_i^T [h,f]: Q[k][n] = B_i^T[n][k] is k-contiguous as it stands
    TPMLP_TRY(record(ev, 3, st));
    if (!H)
      TPMLP_HIP((run_gemm<S, true, true, true>(s.dtype, Tn, h, f, Z, f, B, f, EpiStore<S>{(T*)Yp, h}, st)));
    else
      TPMLP_HIP((run_gemm<S, true, true, false>(s.dtype, Tn, h, f, H, f, B, f, EpiStore<S>{(T*)Yp, h}, st,
                                                room ? reinterpret_cast<float*>(wsb + w.tail_off) : nullptr,
                                                room ? w.tail_bytes : 0)));
  } else if (!H) {
    TPMLP_TRY(record(ev, 3, st));
    TPMLP_HIP((run_gemm<S, true, false, true>(s.dtype, Tn, h, f, Z, f, B, h, EpiStore<S>{(T*)Yp, h}, st)));
  } else if (room && w.bt) {
    TPMLP_HIP((run_transpose<S, false>(B, wsb + w.bt_off, f, h, st)));
    TPMLP_TRY(record(ev, 3, st));
    TPMLP_HIP((run_gemm<S, true, true, false>(s.dtype, Tn, h, f, H, f, wsb + w.bt_off, staged_ld(f),
                                              EpiStore<S>{(T*)Yp, h},
                                              st, reinterpret_cast<float*>(wsb + w.tail_off), w.tail_bytes)));
  } else {
    TPMLP_TRY(record(ev, 3, st));
    TPMLP_HIP((run_gemm<S, true, false, false>(s.dtype, Tn, h, f, H, f, B, h, EpiStore<S>{(T*)Yp, h}, st,
                                               room ? reinterpret_cast<float*>(wsb + w.tail_off) : nullptr,
                                               room ? w.tail_bytes : 0)));
  }
  TPMLP_TRY(record(ev, 4, st));
  return TPMLP_OK;
}

// ACC: dA, dB and db1 are fp32 main gradients that the weight gradients are
// added to (beta = 1) instead of storage-dtype outputs.
template <class S, bool ACC>
int bwd_impl(const tpmlp_shape& s, const void* dY, const void* X, const void* A, const void* B, const void* Z,
             const void* H, void* dZ, void* dXp, void* dA, void* dB, void* db1, const BwdWs& w, void* ws,
             size_t ws_bytes, hipStream_t st, void* const* ev) {
  using T = typename S::T;
  const int64_t Tn = s.tokens, h = s.hidden, f = s.ffn_shard;
  const bool bt = b_t(s);
  // dB [f][h], or [h][f] when B_i^T is given
  auto epi_dB = [&]() {
    if constexpr (ACC) return EpiAccumF32<S>{static_cast<float*>(dB), bt ? f : h};
    else return EpiStore<S>{static_cast<T*>(dB), bt ? f : h};
  };
  auto epi_dA = [&]() {
    if constexpr (ACC) return EpiAccumF32<S>{static_cast<float*>(dA), f};
    else return EpiStore<S>{static_cast<T*>(dA), f};
  };
  char* wsb = static_cast<char*>(ws);
  if (!dZ && w.dz_bytes) dZ = wsb + w.dz_off;
  float* part = w.part_bytes ? reinterpret_cast<float*>(wsb + w.part_off) : nullptr;
  const bool room = ws_bytes >= w.total;
  float* const tail = room ? reinterpret_cast<float*>(wsb + w.tail_off) : nullptr;
  const size_t tcap = room ? w.tail_bytes : 0;

  TPMLP_TRY(record(ev, 0, st));
  // B1: dZ = (dY B_i^T) * gelu'(Z), plus per-tile column sums; Q[k][n] = B_i[n][k] is k-contiguous.
  // With B_i^T [h,f] given, Q[k][n] = B_i^T[k][n] is n-contiguous: it is read
  // in place, or from a k-contiguous copy B_i [f][h + pad] staged first.
  if (!bt) {
    TPMLP_HIP((run_gemm<S, true, true, false>(s.dtype, Tn, f, h, dY, h, B, h,
                                              EpiGeluGrad<S>{(const T*)Z, (T*)dZ, part, f}, st)));
  } else if (room && w.stage_b1) {
    TPMLP_HIP((run_transpose<S, false>(B, wsb + w.bs_off, h, f, st)));
    TPMLP_HIP((run_gemm<S, true, true, false>(s.dtype, Tn, f, h, dY, h, wsb + w.bs_off, staged_ld(h),
                                              EpiGeluGrad<S>{(const T*)Z, (T*)dZ, part, f}, st)));
  } else {
    TPMLP_HIP((run_gemm<S, true, false, false>(s.dtype, Tn, f, h, dY, h, B, f,
                                               EpiGeluGrad<S>{(const T*)Z, (T*)dZ, part, f}, st)));
  }
  TPMLP_TRY(record(ev, 1, st));
  // B5: db1 = sum of the column partials
  if (f > 0) {
    hipLaunchKernelGGL((db1_finish_kernel<S, ACC>), dim3((unsigned)ceil_div(f, 32)), dim3(256), 0, st, part,
                       w.part_tiles, f, db1);
    TPMLP_HIP(hipGetLastError());
  }
  TPMLP_TRY(record(ev, 2, st));
  // TH, TdY + B2: dB = H^T dY. Staged: P = H^T [f,T] (gelu(Z)^T when H is
  // not kept) and Q[k][n] = dY^T[n][k], both k-contiguous. In place: both
  // operands mn-contiguous (and gelu applied to Z on load without H).
  if (room && w.stage_b2) {
    if (H)
      TPMLP_HIP((run_transpose<S, false>(H, wsb + w.ht_off, Tn, f, st)));
    else
      TPMLP_HIP((run_transpose<S, true>(Z, wsb + w.ht_off, Tn, f, st)));
    TPMLP_TRY(record(ev, 3, st));
    TPMLP_HIP((run_transpose<S, false>(dY, wsb + w.dyt_off, Tn, h, st)));
    TPMLP_TRY(record(ev, 4, st));
    if (bt)  // dB^T = dY^T H: the same staged operands, swapped
      TPMLP_HIP((run_gemm<S, true, true, false>(s.dtype, h, f, Tn, wsb + w.dyt_off, staged_ld(Tn), wsb + w.ht_off,
                                                staged_ld(Tn), epi_dB(), st, tail, tcap)));
    else
      TPMLP_HIP((run_gemm<S, true, true, false>(s.dtype, f, h, Tn, wsb + w.ht_off, staged_ld(Tn), wsb + w.dyt_off,
                                                staged_ld(Tn), epi_dB(), st, tail, tcap)));
  } else {
    TPMLP_TRY(record(ev, 3, st));
    TPMLP_TRY(record(ev, 4, st));
    if (bt && H)  // dB^T [h,f] = dY^T H: P[m][k] = dY[k][m], Q[k][n] = H[k][n]
      TPMLP_HIP((run_gemm<S, false, false, false>(s.dtype, h, f, Tn, dY, h, H, f, epi_dB(), st, tail, tcap)));
    else if (bt)  // gelu applies to P only: compute H^T dY with gelu(Z) on load, store it transposed
      TPMLP_HIP((run_gemm<S, false, false, true>(s.dtype, f, h, Tn, Z, f, dY, h,
                                                 EpiTransposed<decltype(epi_dB())>{epi_dB()}, st)));
    else if (H)
      TPMLP_HIP(
          (run_gemm<S, false, false, false>(s.dtype, f, h, Tn, H, f, dY, h, epi_dB(), st, tail, tcap)));
    else
      TPMLP_HIP((run_gemm<S, false, false, true>(s.dtype, f, h, Tn, Z, f, dY, h, epi_dB(), st)));
  }
  TPMLP_TRY(record(ev, 5, st));
  // TX, TdZ + B3: dA = X^T dZ. Staged: P = X^T [h,T], Q[k][n] = dZ^T[n][k].
  if (room && w.stage_b3) {
    TPMLP_HIP((run_transpose<S, false>(X, wsb + w.xt_off, Tn, h, st)));
    TPMLP_TRY(record(ev, 6, st));
    TPMLP_HIP((run_transpose<S, false>(dZ, wsb + w.dzt_off, Tn, f, st)));
    TPMLP_TRY(record(ev, 7, st));
    TPMLP_HIP((run_gemm<S, true, true, false>(s.dtype, h, f, Tn, wsb + w.xt_off, staged_ld(Tn), wsb + w.dzt_off,
                                              staged_ld(Tn),
                                              epi_dA(), st, tail, tcap)));
  } else {
    TPMLP_TRY(record(ev, 6, st));
    TPMLP_TRY(record(ev, 7, st));
    TPMLP_HIP(
        (run_gemm<S, false, false, false>(s.dtype, h, f, Tn, X, h, dZ, f, epi_dA(), st, tail, tcap)));
  }
  TPMLP_TRY(record(ev, 8, st));
  // B4: dXp = dZ A_i^T; Q[k=f][n=h] = A_i[n][k] is k-contiguous
  TPMLP_HIP((run_gemm<S, true, true, false>(s.dtype, Tn, h, f, dZ, f, A, f, EpiStore<S>{(T*)dXp, h}, st, tail, tcap)));
  TPMLP_TRY(record(ev, 9, st));
  return TPMLP_OK;
}

}  // namespace

template <class S, bool PK, bool QK>
static hipError_t planned_gemm_t(int dtype, int64_t M, int64_t N, int64_t K, const void* p, int64_t ldp,
                                 const void* q, int64_t ldq, void* out, int64_t ldo, const void* bias,
                                 float* tail_ws, size_t tail_cap, hipStream_t st) {
  using T = typename S::T;
  if (bias)
    return run_gemm<S, PK, QK, false>(dtype, M, N, K, p, ldp, q, ldq,
                                      EpiBiasGelu<S>{static_cast<const T*>(bias), static_cast<T*>(out), nullptr, ldo},
                                      st);
  return run_gemm<S, PK, QK, false>(dtype, M, N, K, p, ldp, q, ldq, EpiStore<S>{static_cast<T*>(out), ldo}, st,
                                    tail_ws, tail_cap);
}

template <class S>
static hipError_t planned_gemm_s(int dtype, bool pk, bool qk, int64_t M, int64_t N, int64_t K, const void* p,
                                 int64_t ldp, const void* q, int64_t ldq, void* out, int64_t ldo, const void* bias,
                                 float* tail_ws, size_t tail_cap, hipStream_t st) {
  if (pk && qk) return planned_gemm_t<S, true, true>(dtype, M, N, K, p, ldp, q, ldq, out, ldo, bias, tail_ws, tail_cap, st);
  if (pk) return planned_gemm_t<S, true, false>(dtype, M, N, K, p, ldp, q, ldq, out, ldo, bias, tail_ws, tail_cap, st);
  if (qk) return planned_gemm_t<S, false, true>(dtype, M, N, K, p, ldp, q, ldq, out, ldo, bias, tail_ws, tail_cap, st);
  return planned_gemm_t<S, false, false>(dtype, M, N, K, p, ldp, q, ldq, out, ldo, bias, tail_ws, tail_cap, st);
}

hipError_t planned_gemm(int dtype, bool pk, bool qk, int64_t M, int64_t N, int64_t K, const void* p, int64_t ldp,
                        const void* q, int64_t ldq, void* out, int64_t ldo, const void* bias, float* tail_ws,
                        size_t tail_cap, hipStream_t st) {
  if (dtype == TPMLP_F16)
    return planned_gemm_s<StoreF16>(dtype, pk, qk, M, N, K, p, ldp, q, ldq, out, ldo, bias, tail_ws, tail_cap, st);
  if (dtype == TPMLP_BF16)
    return planned_gemm_s<StoreBF16>(dtype, pk, qk, M, N, K, p, ldp, q, ldq, out, ldo, bias, tail_ws, tail_cap, st);
  return hipErrorInvalidValue;
}

size_t planned_gemm_tail_bytes(int dtype, int64_t M, int64_t N, int64_t K, bool kc) {
  return gemm_tail_bytes(dtype, M, N, K, kc);
}

}  // namespace tpmlp

using namespace tpmlp;

extern "C" {

int tp_mlp_abi_version(void) { return TPMLP_ABI_VERSION; }

const char* tp_mlp_status_string(int status) {
  switch (status) {
    case TPMLP_OK: return "ok";
    case TPMLP_ERR_NULL: return "a required pointer is NULL";
    case TPMLP_ERR_SHAPE: return "invalid shape";
    case TPMLP_ERR_ALIGN: return "pointer not 16-byte aligned or dimension not a multiple of 8 (4 for fp32)";
    case TPMLP_ERR_DTYPE: return "unknown dtype";
    case TPMLP_ERR_WORKSPACE: return "workspace too small";
    case TPMLP_ERR_HIP: return "HIP error";
    case TPMLP_ERR_ALIAS: return "an output overlaps an input or another output";
    case TPMLP_ERR_SCRATCH: return "shape needs more than the static scratch (TPMLP_STATIC_SCRATCH_BYTES) holds";
    default: return "unknown status";
  }
}

size_t tp_mlp_fwd_workspace_bytes(const tpmlp_shape* shape) {
  if (check_shape(shape) != TPMLP_OK) return 0;
  return fwd_ws(*shape).total;
}

size_t tp_mlp_workspace_bytes(const tpmlp_shape* shape, unsigned flags) {
  if (check_shape(shape) != TPMLP_OK) return 0;
  const BwdWs w = bwd_ws(*shape, (flags & TPMLP_WS_DZ) != 0);
  const size_t rc = (flags & TPMLP_WS_RECOMPUTE) ? rc_ws(*shape).bytes : 0;
  return rc + ((flags & TPMLP_WS_MINIMAL) ? w.minimal : w.total);
}

int tp_mlp_fwd(const tpmlp_shape* shape, const void* X, const void* A, const void* b1, const void* B, void* Z,
               void* H, void* Yp, void* ws, size_t ws_bytes, void* stream, void* const* events) {
  TPMLP_TRY(check_shape(shape));
  const tpmlp_shape& s = *shape;
  const size_t e = elt_size(s.dtype);
  const size_t Th = (size_t)(s.tokens * s.hidden) * e, hf = (size_t)(s.hidden * s.ffn_shard) * e,
               Tf = (size_t)(s.tokens * s.ffn_shard) * e, fb = (size_t)s.ffn_shard * e;
  const Span in[4] = {{X, Th}, {A, hf}, {b1, fb}, {B, hf}};
  const bool in_req[4] = {true, true, true, true};
  const Span out[4] = {{Z, Tf}, {H, Tf}, {Yp, Th}, {ws, ws ? ws_bytes : 0}};
  const bool out_req[4] = {true, false, true, false};
  TPMLP_TRY(check_buffers(in, 4, in_req, out, 4, out_req));
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (s.dtype) {
    case TPMLP_F32: return fwd_impl<StoreF32>(s, X, A, b1, B, Z, H, Yp, ws, ws_bytes, st, events);
    case TPMLP_F16: return fwd_impl<StoreF16>(s, X, A, b1, B, Z, H, Yp, ws, ws_bytes, st, events);
    default: return fwd_impl<StoreBF16>(s, X, A, b1, B, Z, H, Yp, ws, ws_bytes, st, events);
  }
}

int tp_mlp_bwd(const tpmlp_shape* shape, const void* dY, const void* X, const void* A, const void* B,
               const void* Z, const void* H, void* dZ, void* dXp, void* dA, void* dB, void* db1, void* ws,
               size_t ws_bytes, void* stream, void* const* events) {
  TPMLP_TRY(check_shape(shape));
  const tpmlp_shape& s = *shape;
  const size_t e = elt_size(s.dtype);
  const size_t Th = (size_t)(s.tokens * s.hidden) * e, hf = (size_t)(s.hidden * s.ffn_shard) * e,
               Tf = (size_t)(s.tokens * s.ffn_shard) * e, fb = (size_t)s.ffn_shard * e;
  const BwdWs w = bwd_ws(s, dZ == nullptr);
  const size_t ws_used = ws_bytes >= w.total ? w.total : w.minimal;
  const Span in[6] = {{dY, Th}, {X, Th}, {A, hf}, {B, hf}, {Z, Tf}, {H, Tf}};
  const bool in_req[6] = {true, true, true, true, true, false};
  const Span out[6] = {{dZ, Tf}, {dXp, Th}, {dA, hf}, {dB, hf}, {db1, fb}, {ws, ws_used}};
  const bool out_req[6] = {false, true, true, true, true, true};
  TPMLP_TRY(check_buffers(in, 6, in_req, out, 6, out_req));
  if (ws_bytes < w.minimal) return TPMLP_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (s.dtype) {
    case TPMLP_F32:
      return bwd_impl<StoreF32, false>(s, dY, X, A, B, Z, H, dZ, dXp, dA, dB, db1, w, ws, ws_bytes, st, events);
    case TPMLP_F16:
      return bwd_impl<StoreF16, false>(s, dY, X, A, B, Z, H, dZ, dXp, dA, dB, db1, w, ws, ws_bytes, st, events);
    default:
      return bwd_impl<StoreBF16, false>(s, dY, X, A, B, Z, H, dZ, dXp, dA, dB, db1, w, ws, ws_bytes, st, events);
  }
}

int tp_mlp_bwd_static(const tpmlp_shape* shape, const void* dY, const void* X, const void* A, const void* B,
                      const void* Z, const void* H, void* dZ, void* dXp, void* dA, void* dB, void* db1, void* stream,
                      void* const* events) {
  TPMLP_TRY(check_shape(shape));
  const tpmlp_shape& s = *shape;
  const size_t e = elt_size(s.dtype);
  const size_t Th = (size_t)(s.tokens * s.hidden) * e, hf = (size_t)(s.hidden * s.ffn_shard) * e,
               Tf = (size_t)(s.tokens * s.ffn_shard) * e, fb = (size_t)s.ffn_shard * e;
  const BwdWs w = bwd_ws(s, false);
  const Span in[6] = {{dY, Th}, {X, Th}, {A, hf}, {B, hf}, {Z, Tf}, {H, Tf}};
  const bool in_req[6] = {true, true, true, true, true, false};
  const Span out[5] = {{dZ, Tf}, {dXp, Th}, {dA, hf}, {dB, hf}, {db1, fb}};
  const bool out_req[5] = {true, true, true, true, true};
  TPMLP_TRY(check_buffers(in, 6, in_req, out, 5, out_req));
  if (Tf && !dZ) return TPMLP_ERR_NULL;
  if (w.minimal > TPMLP_STATIC_SCRATCH_BYTES) return TPMLP_ERR_SCRATCH;
  void* ws = nullptr;
  if (w.minimal) TPMLP_TRY(static_scratch(&ws));
  // With exactly the minimal size the plan is tp_mlp_bwd's minimal one:
  // operands read in place, no staged copies, no k-split partials.
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (s.dtype) {
    case TPMLP_F32:
      return bwd_impl<StoreF32, false>(s, dY, X, A, B, Z, H, dZ, dXp, dA, dB, db1, w, ws, w.minimal, st, events);
    case TPMLP_F16:
      return bwd_impl<StoreF16, false>(s, dY, X, A, B, Z, H, dZ, dXp, dA, dB, db1, w, ws, w.minimal, st, events);
    default:
      return bwd_impl<StoreBF16, false>(s, dY, X, A, B, Z, H, dZ, dXp, dA, dB, db1, w, ws, w.minimal, st, events);
  }
}

int tp_mlp_bwd_main_grad(const tpmlp_shape* shape, const void* dY, const void* X, const void* A, const void* B,
                         const void* Z, const void* H, void* dZ, void* dXp, float* dA_main, float* dB_main,
                         float* db1_main, void* ws, size_t ws_bytes, void* stream, void* const* events) {
  TPMLP_TRY(check_shape(shape));
  const tpmlp_shape& s = *shape;
  const size_t e = elt_size(s.dtype);
  const size_t Th = (size_t)(s.tokens * s.hidden) * e, hf = (size_t)(s.hidden * s.ffn_shard) * e,
               Tf = (size_t)(s.tokens * s.ffn_shard) * e;
  const size_t hf4 = (size_t)(s.hidden * s.ffn_shard) * 4, f4 = (size_t)s.ffn_shard * 4;
  const BwdWs w = bwd_ws(s, dZ == nullptr);
  const size_t ws_used = ws_bytes >= w.total ? w.total : w.minimal;
  const Span in[6] = {{dY, Th}, {X, Th}, {A, hf}, {B, hf}, {Z, Tf}, {H, Tf}};
  const bool in_req[6] = {true, true, true, true, true, false};
  const Span out[6] = {{dZ, Tf}, {dXp, Th}, {dA_main, hf4}, {dB_main, hf4}, {db1_main, f4}, {ws, ws_used}};
  const bool out_req[6] = {false, true, true, true, true, true};
  TPMLP_TRY(check_buffers(in, 6, in_req, out, 6, out_req));
  if (ws_bytes < w.minimal) return TPMLP_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (s.dtype) {
    case TPMLP_F32:
      return bwd_impl<StoreF32, true>(s, dY, X, A, B, Z, H, dZ, dXp, dA_main, dB_main, db1_main, w, ws, ws_bytes, st,
                                      events);
    case TPMLP_F16:
      return bwd_impl<StoreF16, true>(s, dY, X, A, B, Z, H, dZ, dXp, dA_main, dB_main, db1_main, w, ws, ws_bytes, st,
                                      events);
    default:
      return bwd_impl<StoreBF16, true>(s, dY, X, A, B, Z, H, dZ, dXp, dA_main, dB_main, db1_main, w, ws, ws_bytes,
                                       st, events);
  }
}

int tp_mlp_bwd_recompute(const tpmlp_shape* shape, const void* dY, const void* X, const void* A, const void* b1,
                         const void* B, void* dZ, void* dXp, void* dA, void* dB, void* db1, void* ws,
                         size_t ws_bytes, void* stream, void* const* events) {
  TPMLP_TRY(check_shape(shape));
  const tpmlp_shape& s = *shape;
  const size_t e = elt_size(s.dtype);
  const size_t Th = (size_t)(s.tokens * s.hidden) * e, hf = (size_t)(s.hidden * s.ffn_shard) * e,
               Tf = (size_t)(s.tokens * s.ffn_shard) * e, fb = (size_t)s.ffn_shard * e;
  const RcWs r = rc_ws(s);
  const BwdWs w = bwd_ws(s, dZ == nullptr);
  const size_t rest = ws_bytes > r.bytes ? ws_bytes - r.bytes : 0;
  const size_t ws_used = r.bytes + (rest >= w.total ? w.total : w.minimal);
  const Span in[5] = {{dY, Th}, {X, Th}, {A, hf}, {b1, fb}, {B, hf}};
  const bool in_req[5] = {true, true, true, true, true};
  const Span out[6] = {{dZ, Tf}, {dXp, Th}, {dA, hf}, {dB, hf}, {db1, fb}, {ws, ws_used}};
  const bool out_req[6] = {false, true, true, true, true, true};
  TPMLP_TRY(check_buffers(in, 5, in_req, out, 6, out_req));
  if (ws_bytes < r.bytes + w.minimal) return TPMLP_ERR_WORKSPACE;
  char* wsb = static_cast<char*>(ws);
  void* Z = wsb;  // Z_i recomputed at the front of the workspace
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* const* ev_b = events ? events + 2 : nullptr;
  switch (s.dtype) {
    case TPMLP_F32:
      TPMLP_TRY(recompute_z<StoreF32>(s, X, A, b1, Z, r, wsb, st, events));
      return bwd_impl<StoreF32, false>(s, dY, X, A, B, Z, nullptr, dZ, dXp, dA, dB, db1, w, wsb + r.bytes, rest, st,
                                       ev_b);
    case TPMLP_F16:
      TPMLP_TRY(recompute_z<StoreF16>(s, X, A, b1, Z, r, wsb, st, events));
      return bwd_impl<StoreF16, false>(s, dY, X, A, B, Z, nullptr, dZ, dXp, dA, dB, db1, w, wsb + r.bytes, rest, st,
                                       ev_b);
    default:
      TPMLP_TRY(recompute_z<StoreBF16>(s, X, A, b1, Z, r, wsb, st, events));
      return bwd_impl<StoreBF16, false>(s, dY, X, A, B, Z, nullptr, dZ, dXp, dA, dB, db1, w, wsb + r.bytes, rest,
                                        st, ev_b);
  }
}

size_t tp_mlp_db2_workspace_bytes(const tpmlp_shape* shape) {
  if (check_shape(shape) != TPMLP_OK || shape->dtype == TPMLP_F32) return 0;
  return (size_t)ceil_div(shape->tokens, 256) * (size_t)shape->hidden * sizeof(float);
}

int tp_mlp_db2(const tpmlp_shape* shape, const void* dY, void* db2, int accumulate, void* ws, size_t ws_bytes,
               void* stream) {
  TPMLP_TRY(check_shape(shape));
  const tpmlp_shape& s = *shape;
  if (ceil_div(s.tokens, 256) > 65535) return TPMLP_ERR_SHAPE;  // grid y of the first pass
  const size_t e = elt_size(s.dtype);
  const size_t need = tp_mlp_db2_workspace_bytes(shape);
  const size_t ob = (size_t)s.hidden * (accumulate ? sizeof(float) : e);
  const Span in[1] = {{dY, (size_t)(s.tokens * s.hidden) * e}};
  const bool in_req[1] = {true};
  const Span out[2] = {{db2, ob}, {ws, std::min(need, ws_bytes)}};
  const bool out_req[2] = {true, need > 0};
  TPMLP_TRY(check_buffers(in, 1, in_req, out, 2, out_req));
  if (ws_bytes < need) return TPMLP_ERR_WORKSPACE;
  if (s.hidden == 0) return TPMLP_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const unsigned gx = (unsigned)ceil_div(s.hidden, 256);
  if (s.dtype == TPMLP_F32) {
    if (accumulate)
      hipLaunchKernelGGL(colsum_f32_kernel<true>, dim3(gx), dim3(256), 0, st, static_cast<const float*>(dY), s.tokens,
                         s.hidden, static_cast<float*>(db2));
    else
      hipLaunchKernelGGL(colsum_f32_kernel<false>, dim3(gx), dim3(256), 0, st, static_cast<const float*>(dY),
                         s.tokens, s.hidden, static_cast<float*>(db2));
    return hipGetLastError() == hipSuccess ? TPMLP_OK : TPMLP_ERR_HIP;
  }
  const int nblk = (int)ceil_div(s.tokens, 256);
  float* part = static_cast<float*>(ws);
  if (nblk > 0) {
    if (s.dtype == TPMLP_F16)
      hipLaunchKernelGGL(colsum_part_kernel<StoreF16>, dim3(gx, (unsigned)nblk), dim3(256), 0, st,
                         static_cast<const uint16_t*>(dY), s.tokens, s.hidden, part);
    else
      hipLaunchKernelGGL(colsum_part_kernel<StoreBF16>, dim3(gx, (unsigned)nblk), dim3(256), 0, st,
                         static_cast<const uint16_t*>(dY), s.tokens, s.hidden, part);
    TPMLP_HIP(hipGetLastError());
  }
  if (accumulate)
    hipLaunchKernelGGL(colsum_accum_kernel, dim3(gx), dim3(256), 0, st, part, nblk, s.hidden, static_cast<float*>(db2));
  else if (s.dtype == TPMLP_F16)
    hipLaunchKernelGGL(colsum_finish_kernel<StoreF16>, dim3(gx), dim3(256), 0, st, part, nblk, s.hidden,
                       static_cast<uint16_t*>(db2));
  else
    hipLaunchKernelGGL(colsum_finish_kernel<StoreBF16>, dim3(gx), dim3(256), 0, st, part, nblk, s.hidden,
                       static_cast<uint16_t*>(db2));
  return hipGetLastError() == hipSuccess ? TPMLP_OK : TPMLP_ERR_HIP;
}

int tp_mlp_reduce_partials(const tpmlp_shape* shape, int nparts, const void* const* parts, const void* bias,
                           int64_t row_begin, int64_t row_end, void* out, void* stream) {
  TPMLP_TRY(check_shape(shape));
  const tpmlp_shape& s = *shape;
  if (nparts < 1 || nparts > kMaxParts) return TPMLP_ERR_SHAPE;
  if (!parts) return TPMLP_ERR_NULL;
  if (row_begin < 0 || row_end < row_begin || row_end > s.tokens) return TPMLP_ERR_SHAPE;
  const size_t e = elt_size(s.dtype);
  const int64_t rows = row_end - row_begin;
  const size_t Th = (size_t)(s.tokens * s.hidden) * e, hb = (size_t)s.hidden * e, ob = (size_t)(rows * s.hidden) * e;
  Span in[kMaxParts + 1];
  bool in_req[kMaxParts + 1];
  for (int i = 0; i < nparts; ++i) {
    in[i] = Span{parts[i], Th};
    in_req[i] = true;
  }
  in[nparts] = Span{bias, hb};
  in_req[nparts] = false;
  const Span outs[1] = {{out, ob}};
  const bool out_req[1] = {true};
  TPMLP_TRY(check_buffers(in, nparts + 1, in_req, outs, 1, out_req));
  if (ob == 0) return TPMLP_OK;
  PartList pl{};
  for (int i = 0; i < nparts; ++i) pl.p[i] = parts[i];
  const int64_t chunks = rows * s.hidden / (16 / (int64_t)e);
  const unsigned grid = (unsigned)std::min<int64_t>(ceil_div(chunks, 256), int64_t(1) << 20);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (s.dtype) {
    case TPMLP_F32:
      hipLaunchKernelGGL(reduce_partials_kernel<StoreF32>, dim3(grid), dim3(256), 0, st, pl, nparts,
                         static_cast<const float*>(bias), row_begin, rows, s.hidden, static_cast<float*>(out));
      break;
    case TPMLP_F16:
      hipLaunchKernelGGL(reduce_partials_kernel<StoreF16>, dim3(grid), dim3(256), 0, st, pl, nparts,
                         static_cast<const uint16_t*>(bias), row_begin, rows, s.hidden, static_cast<uint16_t*>(out));
      break;
    default:
      hipLaunchKernelGGL(reduce_partials_kernel<StoreBF16>, dim3(grid), dim3(256), 0, st, pl, nparts,
                         static_cast<const uint16_t*>(bias), row_begin, rows, s.hidden, static_cast<uint16_t*>(out));
      break;
  }
  return hipGetLastError() == hipSuccess ? TPMLP_OK : TPMLP_ERR_HIP;
}

int tp_mlp_debug_plan(int tile, int tail_cus) {
  if (tile < TPMLP_PLAN_AUTO || tile > TPMLP_PLAN_DMA320 || tail_cus < 0 || tail_cus > 4096) return TPMLP_ERR_SHAPE;
  g_plan_tile.store(tile, std::memory_order_relaxed);
  g_plan_cus.store(tail_cus, std::memory_order_relaxed);
  return TPMLP_OK;
}

}  // extern "C"
