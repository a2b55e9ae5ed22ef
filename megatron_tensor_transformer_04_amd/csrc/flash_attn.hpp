// Fused attention core for gfx950: scores and probabilities never leave the
// chip. For one sequence b and head j, with Q, K, V the [seq, d] column
// blocks of QKV and x = Q K^T / sqrt(d) (keys after the query masked out
// when causal),
//   forward:  O = softmax(x) V and L = log sum_k exp(x_k) per query row,
//             one 64-key block at a time with a running maximum and sum per
//             row (the online form of the softmax);
//   backward: P = exp(x - L) recomputed from L, then
//             dV = P^T dO, dS = P (dO V^T - D) / sqrt(d), D = rowsum(dO O),
//             dK = dS^T Q (flash_bwd_kv_kernel, one workgroup per 128 keys,
//             one launch for dV and one for dK)
//             and dQ = dS K (flash_bwd_q_kernel, one workgroup per 128
//             queries, recomputing P and dS): every output element is summed
//             by one lane in a fixed order, no atomics.
// P and dS are rounded to the storage dtype before they enter a product, as
// the materialized path rounds its stored P and dS.
//
// Products (v_mfma_f32_32x32x16_{bf16,f16}): lane l = 32 h + c of a wave
// holds A[c][8 h .. 8 h + 7] and B[8 h .. 8 h + 7][c] of the operands and
// C[8 g + 4 h + e][c], g, e = 0..3, of the 32 x 32 result (register 4 g + e).
// Each kernel computes the scores with the lane's own row (query, or key in
// the dK/dV kernel) as the result's column c; the lane then holds 16 of the
// other index per fragment, 4 h + {0..3, 8..11, 16..19, 24..27}. Those
// values, rounded to 16 bits, are directly the B operand of the next product
// over that index: for a 16-wide step, k-slots 8 h + 0..3 carry entries
// 4 h + 0..3 and slots 8 h + 4..7 carry 8 + 4 h + 0..3 (pack_step). The A
// operand of that product takes the same slot order from a row-major tile in
// LDS with two transposing reads (ds_read_b64_tr_b16, frag_cols): the sum
// over k does not depend on the order, and no value moves between lanes.
// Lanes l and l + 32 hold the same row: the forward exchanges the block
// maximum between them once per 32-key fragment and the running sums at the
// end.
//
// Workgroups of eight waves: four row groups of 32 rows, each in two halves
// (waves g and g + 4) that take alternate 64-row blocks of the loop and add
// their partial results through LDS at the end, in a fixed order. The
// longest row block's chain of dependent blocks, which sets a causal
// launch's time, is then half as long.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "numerics.hpp"

namespace tpmlp {
namespace flash {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kThreads = 512;  // eight waves: four row groups of 32, each in two halves
constexpr int kRows = 128;     // rows (queries or keys) per workgroup
constexpr int kBlk = 64;       // keys (queries) per block of the inner loop
constexpr int kStage = 128;    // rows per LDS stage: the blocks of both halves
// The forward's reference maximum moves only when a row's scores exceed it
// by more than this (log2 units): probabilities stay below 2^8.
constexpr float kRescale = 8.0f;

// Row pitch in bytes of a tile of C 16-bit columns in LDS: 16 bytes of
// padding put the 32 rows of a 16-byte fragment read, and the 4 rows of a
// transposing read, on distinct banks.
template <int C>
constexpr int pitch() {
  return C * 2 + 16;
}

// Byte offset past the end of any buffer here: a buffer load from it
// returns zeros.
constexpr uint32_t kOob = 0x80000000u;

// Raw buffer resource over `bytes` bytes at `p` (below 2^31), from
// wave-uniform values so that it lives in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void* p, int64_t bytes) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), 0, n, 0x00020000);
}

// Rows [r0, r0 + R) and columns [0, C) of one head's block of a row-major
// 16-bit matrix (row pitch ld), moved through registers into an LDS tile
// (register-staged, so that the loads of the next block are in flight while
// the current one is computed). The loads are buffer loads over the
// sequence's rows of the head's block: rows past the sequence read as zeros
// from the buffer's range check, columns >= d from an offset past the end.
// Each thread's offsets are fixed (row r0 enters as the scalar offset).
// `one_bits` != 0: column d of every row holds that 16-bit value (the
// forward's column of ones, whose product with P^T is the row sum).
template <int R, int C>
struct TileCopy {
  static constexpr int CH = C / 8, NCH = R * CH, N = (NCH + kThreads - 1) / kThreads;
  uint32_t off[N], one[N];
  u32x4 v[N];
  __device__ __forceinline__ void init(int64_t ld, int d, int tid, uint32_t one_bits = 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + i * kThreads, r = c / CH, cc = c % CH;
      off[i] = c < NCH && cc * 8 < d ? (uint32_t)(r * ld * 2 + cc * 16) : kOob;
      one[i] = c < NCH && cc * 8 == d ? one_bits : 0u;
    }
  }
  // the loaded registers are first touched by store(): no wait in between
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int row_off) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off[i], row_off, 0);
  }
  __device__ __forceinline__ void store(char* t, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + i * kThreads, r = c / CH, cc = c % CH;
      u32x4 x = v[i];
      x[0] |= one[i];
      if (c < NCH) *reinterpret_cast<u32x4*>(t + r * pitch<C>() + cc * 16) = x;
    }
  }
};

// Operand fragment from a row-major tile: row row0 + c, columns
// col0 + 8 h .. + 7 (one 16-byte read).
template <int C>
__device__ __forceinline__ u32x4 frag_rows(const char* t, int row0, int col0, int lane) {
  return *reinterpret_cast<const u32x4*>(t + (row0 + (lane & 31)) * pitch<C>() + (col0 + 8 * (lane >> 5)) * 2);
}

// Transposed operand fragment: column col0 + c of rows
// row0 + {4 h .. 4 h + 3, 8 + 4 h .. 8 + 4 h + 3}, the slot order of
// pack_step. A transposing read takes a 4-row x 16-column block of 16-bit
// values, lane j of each 16 addressing row j / 4, columns 4 (j % 4) .. + 3,
// and returns column j of the block to lane j, rows in order.
template <int C>
__device__ __forceinline__ u32x4 frag_cols(const char* t, int row0, int col0, int lane) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const int g = lane >> 4, j = lane & 15;
  u32x4 out;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int r = row0 + 8 * hh + 4 * (g >> 1) + (j >> 2);
    const int c = col0 + 16 * (g & 1) + 4 * (j & 3);
    const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(t + r * pitch<C>() + c * 2));
    const u32x2 w = __builtin_bit_cast(u32x2, x);
    out[2 * hh] = w[0];
    out[2 * hh + 1] = w[1];
  }
  return out;
}

// B operand of the 16-wide step st (0 or 1) of a 32-entry fragment: values
// v[8 st .. 8 st + 7] rounded to storage, in k-slots 8 h + 0..7.
template <class S>
__device__ __forceinline__ u32x4 pack_step(const f32x16& v, int st) {
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = S::pack2(v[8 * st + 2 * e], v[8 * st + 2 * e + 1]);
  return w;
}

// Row offset, within the 32-entry fragment, of result register r of a lane
// in half h: 8 (r / 4) + 4 h + r % 4.
__device__ __forceinline__ int frag_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Store a 32 x 32 accumulator fragment X^T (rows d0 + .. of the head's
// columns, the result's column = this lane's output row) as 16-bit values
// times `mul`: four consecutive columns per 8-byte store, columns >= d
// skipped.
template <class S>
__device__ __forceinline__ void store_t(uint16_t* orow, const f32x16& x, int d0, int d, int h, float mul) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int dc = d0 + 8 * g + 4 * h;
    if (dc < d) {
      u32x2 w;
      w[0] = S::pack2(x[4 * g] * mul, x[4 * g + 1] * mul);
      w[1] = S::pack2(x[4 * g + 2] * mul, x[4 * g + 3] * mul);
      *reinterpret_cast<u32x2*>(orow + dc) = w;
    }
  }
}

struct Args {
  const uint16_t* qkv;  // [T][3q]: Q | K | V blocks, head j at columns j d .. j d + d - 1 of each
  const uint16_t* dO;   // [T][q] (backward)
  const float* D;       // rowsum(dO O) [batch*heads][seq] (backward)
  float* lse;           // L [batch*heads][seq], natural log (forward: written)
  uint16_t* out;        // forward: O [T][q]; backward: dQKV [T][3q]
  int64_t s, ld3, ldo;  // seq; row pitches of QKV (3q) and of O / dO (q)
  int heads, d, q, nblk, Z;  // nblk: 128-row blocks per sequence; Z = batch * heads
  float scale_log2;          // log2(e) / sqrt(d)
  float scale;               // 1 / sqrt(d)
  int causal;
  uint32_t one_bits;         // 1.0 in the storage format
};

// Largest of the 16 values of a fragment.
__device__ __forceinline__ float frag_max(const f32x16& v) {
  float m0 = fmaxf(fmaxf(v[0], v[1]), v[2]), m1 = fmaxf(fmaxf(v[3], v[4]), v[5]);
  float m2 = fmaxf(fmaxf(v[6], v[7]), v[8]), m3 = fmaxf(fmaxf(v[9], v[10]), v[11]);
  float m4 = fmaxf(fmaxf(v[12], v[13]), v[14]);
  return fmaxf(fmaxf(fmaxf(m0, m1), fmaxf(m2, m3)), fmaxf(m4, v[15]));
}

// The two halves of a row group (waves g and g + 4) take alternate blocks
// of the loop (even and odd), so that the longest row block's chain of
// dependent blocks is half as long; at the end the second half hands its
// accumulators (and two per-lane values) to the first through LDS, which
// adds them in a fixed order. Buffer layout: group g's values at
// buf[g][v][lane], v < FD * 16 + 2.
template <int FD>
__device__ __forceinline__ void half_put(float* buf, int g, int lane, const f32x16 (&x)[FD], float s0, float s1) {
  float* p = buf + g * 64 * (FD * 16 + 2);
#pragma unroll
  for (int f = 0; f < FD; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) p[(f * 16 + r) * 64 + lane] = x[f][r];
  p[FD * 16 * 64 + lane] = s0;
  p[(FD * 16 + 1) * 64 + lane] = s1;
}

template <int FD>
__device__ __forceinline__ void half_get(const float* buf, int g, int lane, f32x16 (&x)[FD], float& s0, float& s1) {
  const float* p = buf + g * 64 * (FD * 16 + 2);
#pragma unroll
  for (int f = 0; f < FD; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) x[f][r] = p[(f * 16 + r) * 64 + lane];
  s0 = p[FD * 16 * 64 + lane];
  s1 = p[(FD * 16 + 1) * 64 + lane];
}

// Forward: one workgroup per (pair z, 128 queries), the last (longest, when
// causal) query blocks first; wave w owns queries q0 + 32 (w % 4) + c and
// the key blocks of parity w / 4. Scores stay in raw units (Q K^T) until
// the exponent, exp2(x c - m c) with c = log2(e) / sqrt(d) in one FMA. m is
// a reference maximum per row and half: it moves, and O and the running sum
// are rescaled by exp2((m_old - m_new) c), only in the blocks where some
// row's scores exceed it by more than kRescale (log2 units).
// ONES (d not a multiple of 32): V's zero padding gets a column of ones at
// d, so that O^T's row d accumulates the row sum of the rounded
// probabilities in the same products (rescaled with O); otherwise the lanes
// add their probabilities.
template <class S, int KS, int FD, bool ONES>
__global__ __launch_bounds__(kThreads) void flash_fwd_kernel(Args a) {
  constexpr int DK = 16 * KS, DV = 32 * FD;
  constexpr int KB = kStage * pitch<DK>(), STG = KB + kStage * pitch<DV>();
  static_assert(4 * 64 * (FD * 16 + 2) * 4 <= 2 * STG, "the halves' exchange fits in the stages");
  __shared__ __attribute__((aligned(16))) char smem[2 * STG];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, g = wave & 3, hk = wave >> 2;
  const int qb = a.nblk - 1 - (int)(blockIdx.x / a.Z), z = (int)(blockIdx.x % a.Z);
  const int b = z / a.heads, j = z % a.heads;
  const int64_t q0 = (int64_t)qb * kRows, qw = q0 + 32 * g, qi = qw + (lane & 31);
  const uint16_t* Qp = a.qkv + (int64_t)b * a.s * a.ld3 + (int64_t)j * a.d;
  const uint16_t* Kp = Qp + a.q;
  const uint16_t* Vp = Qp + 2 * a.q;
  const int64_t kv_end = a.causal ? min(a.s, q0 + kRows) : a.s;
  const int nit = (int)((kv_end + kStage - 1) / kStage);
  // keys this wave reads: none if all its queries are past the end, else up
  // to its last query when causal (wave-uniform)
  const int64_t wave_kend = qw >= a.s ? 0 : (a.causal ? min(kv_end, qw + 32) : kv_end);
  const uint32_t ones = ONES ? a.one_bits : 0u;
  const float c = a.scale_log2;

  u32x4 qf[KS];  // B operand of K Q^T: query qi, columns 16 ks + 8 h .. + 7
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int dd = 16 * ks + 8 * h;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (qi < a.s && dd < a.d) v = *reinterpret_cast<const u32x4*>(Qp + qi * a.ld3 + dd);
    qf[ks] = v;
  }
  const int rowb = (int)(a.ld3 * 2);
  const auto krs = wave_rsrc(Kp, (a.s * a.ld3 - (int64_t)j * a.d - a.q) * 2);
  const auto vrs = wave_rsrc(Vp, (a.s * a.ld3 - (int64_t)j * a.d - 2 * a.q) * 2);
  TileCopy<kStage, DK> kt;
  TileCopy<kStage, DV> vt;
  kt.init(a.ld3, a.d, tid);
  vt.init(a.ld3, a.d, tid, ones);
  f32x16 o[FD];
#pragma unroll
  for (int f = 0; f < FD; ++f) o[f] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;

  if (nit > 0) {
    kt.load(krs, 0);
    vt.load(vrs, 0);
    kt.store(smem, tid);
    vt.store(smem + KB, tid);
  }
  // every load issued so far (the Q fragments too) has landed: the loop's
  // products then wait only for their own LDS reads, not for the next
  // stage's loads in flight
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int it = 0; it < nit; ++it) {
    // the next stage's tiles (past the end in the last iteration: zeros,
    // stored to the stage nothing reads any more)
    kt.load(krs, (it + 1) * kStage * rowb);
    vt.load(vrs, (it + 1) * kStage * rowb);
    const int64_t k0 = (int64_t)it * kStage + hk * kBlk;  // this half's block
    if (k0 < wave_kend) {
      const char* sk = smem + (it & 1) * STG + hk * kBlk * pitch<DK>();
      const char* sv = smem + (it & 1) * STG + KB + hk * kBlk * pitch<DV>();
      // x^T = K Q^T (raw): keys k0 + 32 mf + frag_row(r, h), query qi. All
      // of the block's K fragments are read before the first product, and
      // V's right after the last, so that the LDS latency is paid once per
      // phase (the V reads land while the softmax runs).
      u32x4 kfr[2][KS];
#pragma unroll
      for (int mf = 0; mf < 2; ++mf)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kfr[mf][ks] = frag_rows<DK>(sk, 32 * mf, 16 * ks, lane);
      // fragment 0's products first, then fragment 1's: the softmax of
      // fragment 0 then runs while fragment 1's products execute, and that
      // of fragment 1 while fragment 0's P V products do
      f32x16 sc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int mf = 0; mf < 2; ++mf)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sc[mf] = S::mfma32x32x16(kfr[mf][ks], qf[ks], sc[mf]);
      // (V read ahead only while its 16 FD registers fit beside the rest)
      constexpr bool kVAhead = FD <= 3;
      u32x4 vfr[4][FD];
      if constexpr (kVAhead) {
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int f = 0; f < FD; ++f) vfr[st][f] = frag_cols<DV>(sv, 16 * st, 32 * f, lane);
      }
      // keys past the end, or after the query: only in the last block and on
      // the diagonal (wave-uniform)
      const bool masked = k0 + kBlk > a.s || (a.causal && k0 + kBlk - 1 > qw);
      // one 32-key fragment at a time: its maximum and the reference update,
      // its probabilities, then its two 16-key steps of O^T += V^T P^T
#pragma unroll
      for (int mf = 0; mf < 2; ++mf) {
        if (masked) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t ki = k0 + 32 * mf + frag_row(r, h);
            if (ki >= a.s || (a.causal && ki > qi)) sc[mf][r] = -INFINITY;
          }
        }
        float mb = frag_max(sc[mf]);
        mb = fmaxf(mb, __shfl_xor(mb, 32));
        // the first fragment always sets the reference; p <= 2^kRescale after
        if (__ballot((mb - m_run) * c > kRescale)) {
          const float m_new = fmaxf(m_run, mb);
          // m_new stays -inf only while every key seen is masked: nothing to rescale then
          const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f((m_run - m_new) * c);
#pragma unroll
          for (int f = 0; f < FD; ++f) o[f] *= alpha;
          if (!ONES) l_run *= alpha;
          m_run = m_new;
        }
        const float mc = m_run == -INFINITY ? 0.0f : m_run * c;
        float ls = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[mf][r], c, -mc));
          sc[mf][r] = p;
          if (!ONES) ls += p;
        }
        if (!ONES) l_run += ls;
#pragma unroll
        for (int st = 2 * mf; st < 2 * mf + 2; ++st) {
          const u32x4 pf = pack_step<S>(sc[mf], st & 1);
#pragma unroll
          for (int f = 0; f < FD; ++f)
            o[f] = S::mfma32x32x16(kVAhead ? vfr[st][f] : frag_cols<DV>(sv, 16 * st, 32 * f, lane), pf, o[f]);
        }
      }
    }
    // the other stage was last read in the previous iteration, before the
    // barrier that ended it
    {
      char* nx = smem + ((it + 1) & 1) * STG;
      kt.store(nx, tid);
      vt.store(nx + KB, tid);
    }
    __syncthreads();
  }

  // the second half's O^T, reference maximum and sum to the first; every
  // stage read is done (the loop's last barrier)
  float* xbuf = reinterpret_cast<float*>(smem);
  if (hk == 1) half_put<FD>(xbuf, g, lane, o, m_run, l_run);
  __syncthreads();
  if (hk == 1) return;
  {
    f32x16 o2[FD];
    float m2, l2;
    half_get<FD>(xbuf, g, lane, o2, m2, l2);
    const float m = fmaxf(m_run, m2);
    const float fa = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m_run - m) * c);
    const float fb = m2 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m2 - m) * c);
#pragma unroll
    for (int f = 0; f < FD; ++f) o[f] = o[f] * fa + o2[f] * fb;
    l_run = l_run * fa + l2 * fb;
    m_run = m;
  }
  // the row sum: O^T's row d (in lanes h = 0, register 4 g1 of the last
  // fragment), or the two lane halves' sums
  float l_all;
  if (ONES) {
    const int g1 = (a.d - 32 * (FD - 1)) >> 3;
    const f32x16& ol = o[FD - 1];
    const float lv = g1 == 1 ? ol[4] : (g1 == 2 ? ol[8] : ol[12]);
    l_all = __shfl(lv, lane & 31);
  } else {
    l_all = l_run + __shfl_xor(l_run, 32);
  }
  // O = O^T / l (rows d < a.d); L = (m c + log2 l) ln 2
  if (qi < a.s) {
    const float inv = 1.0f / l_all;
    uint16_t* orow = a.out + ((int64_t)b * a.s + qi) * a.ldo + (int64_t)j * a.d;
#pragma unroll
    for (int f = 0; f < FD; ++f) store_t<S>(orow, o[f], 32 * f, a.d, h, inv);
    if (h == 0) a.lse[(int64_t)z * a.s + qi] = (m_run * c + log2f(l_all)) * kLn2;
  }
}

// dV (ROLE_DK false) or dK (ROLE_DK true): one workgroup per (pair z, 128
// keys), the first (longest, when causal) key blocks first; wave w owns keys
// k0 + 32 (w % 4) + c and the query blocks of parity w / 4 (Q and dO tiles,
// and per query L log2(e) and D / sqrt(d), in LDS):
//   p = exp2(x c - L log2(e));  dV^T += dO^T P;
//   dS = p (dP / sqrt(d) - D / sqrt(d)), dP = dO V^T;  dK^T += Q^T dS.
// The two gradients are separate launches that both recompute the scores:
// each then holds one d-wide accumulator.
template <class S, int KS, int FD, bool ROLE_DK>
__global__ __launch_bounds__(kThreads) void flash_bwd_kv_kernel(Args a) {
  constexpr int DV = 32 * FD;
  constexpr int TB = kStage * pitch<DV>(), STG = 2 * TB + 2 * kStage * 4;
  static_assert(4 * 64 * (FD * 16 + 2) * 4 <= 2 * STG, "the halves' exchange fits in the stages");
  __shared__ __attribute__((aligned(16))) char smem[2 * STG];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, g = wave & 3, hq = wave >> 2;
  const int kblk = (int)(blockIdx.x / a.Z), z = (int)(blockIdx.x % a.Z);
  const int b = z / a.heads, j = z % a.heads;
  const int64_t k0 = (int64_t)kblk * kRows, kw = k0 + 32 * g, ki = kw + (lane & 31);
  const uint16_t* Qp = a.qkv + (int64_t)b * a.s * a.ld3 + (int64_t)j * a.d;
  const uint16_t* Kp = Qp + a.q;
  const uint16_t* Vp = Qp + 2 * a.q;
  const uint16_t* dOp = a.dO + (int64_t)b * a.s * a.ldo + (int64_t)j * a.d;
  const float* Lz = a.lse + (int64_t)z * a.s;
  const float* Dz = a.D + (int64_t)z * a.s;
  const int64_t qstart = a.causal ? k0 : 0;  // queries before the block's first key see none of its keys
  const int nit = (int)((a.s - qstart + kStage - 1) / kStage);
  const bool live = kw < a.s;
  const float c = a.scale_log2, sc_d = a.scale;

  u32x4 kf[KS], vf[KS];  // B operands of Q K^T and dO V^T: key ki, columns 16 ks + 8 h .. + 7
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int dd = 16 * ks + 8 * h;
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (ki < a.s && dd < a.d) {
      x = *reinterpret_cast<const u32x4*>(Kp + ki * a.ld3 + dd);
      if (ROLE_DK) y = *reinterpret_cast<const u32x4*>(Vp + ki * a.ld3 + dd);
    }
    kf[ks] = x;
    vf[ks] = y;
  }
  const auto qrs = wave_rsrc(Qp, (a.s * a.ld3 - (int64_t)j * a.d) * 2);
  const auto drs = wave_rsrc(dOp, (a.s * a.ldo - (int64_t)j * a.d) * 2);
  const int rowq = (int)(a.ld3 * 2), rowd = (int)(a.ldo * 2);
  TileCopy<kStage, DV> qt, dt;
  qt.init(a.ld3, a.d, tid);
  dt.init(a.ldo, a.d, tid);
  // thread t < 128: L of query t of the stage (+inf past the end: p = 0);
  // 128 <= t < 256: its D; scaled to L log2(e) and D / sqrt(d) when stored
  float rowv = 0.0f;
  auto load_rows = [&](int64_t r0) {
    const int t = tid & 127;
    if (tid < 128) rowv = r0 + t < a.s ? Lz[r0 + t] : INFINITY;
    else if (ROLE_DK && tid < 256) rowv = r0 + t < a.s ? Dz[r0 + t] : 0.0f;
  };
  auto store_stage = [&](char* t) {
    qt.store(t, tid);
    dt.store(t + TB, tid);
    if (tid < (ROLE_DK ? 256 : 128)) reinterpret_cast<float*>(t + 2 * TB)[tid] = rowv * (tid < 128 ? kLog2e : sc_d);
  };
  f32x16 acc[FD];  // dV^T or dK^T: rows d, column key ki
#pragma unroll
  for (int f = 0; f < FD; ++f) acc[f] = f32x16{};

  if (nit > 0) {
    qt.load(qrs, (int)qstart * rowq);
    dt.load(drs, (int)qstart * rowd);
    load_rows(qstart);
    store_stage(smem);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // as in the forward: nothing in flight before the loop
  __syncthreads();
  for (int it = 0; it < nit; ++it) {
    const int64_t r0 = qstart + (int64_t)it * kStage;
    // the next stage (past the end in the last iteration, as in the forward)
    qt.load(qrs, (int)(r0 + kStage) * rowq);
    dt.load(drs, (int)(r0 + kStage) * rowd);
    load_rows(r0 + kStage);
    const int64_t q0 = r0 + hq * kBlk;  // this half's block
    // causal: a block whose queries all precede the wave's keys has p = 0
    if (live && q0 < a.s && !(a.causal && q0 + kBlk - 1 < kw)) {
      const char* sq = smem + (it & 1) * STG + hq * kBlk * pitch<DV>();
      const char* sd = sq + TB;
      const float* sl = reinterpret_cast<const float*>(smem + (it & 1) * STG + 2 * TB) + hq * kBlk;
      // queries before the wave's last key: only on the diagonal (wave-uniform)
      auto block = [&](auto masked) {
        // one 32-query fragment at a time (mf): x = Q K^T (and dP = dO V^T),
        // rows (queries) q0 + 32 mf + frag_row(r, h), column key ki
#pragma unroll
        for (int mf = 0; mf < 2; ++mf) {
          // the fragment's LDS reads are all issued ahead of its products:
          // Q (and dO) rows first, the transposed operand of the gradient
          // product right after, landing while the softmax part runs
          u32x4 qfr[KS], dfr[KS], tfr[2][FD];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            qfr[ks] = frag_rows<DV>(sq, 32 * mf, 16 * ks, lane);
            if (ROLE_DK) dfr[ks] = frag_rows<DV>(sd, 32 * mf, 16 * ks, lane);
          }
          f32x16 p = f32x16{}, dp = f32x16{};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            p = S::mfma32x32x16(qfr[ks], kf[ks], p);
            if (ROLE_DK) dp = S::mfma32x32x16(dfr[ks], vf[ks], dp);
          }
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int f = 0; f < FD; ++f) tfr[st][f] = frag_cols<DV>(ROLE_DK ? sq : sd, 32 * mf + 16 * st, 32 * f, lane);
#pragma unroll
          for (int gg = 0; gg < 4; ++gg) {
            const int rr = 32 * mf + 8 * gg + 4 * h;
            const f32x4 L4 = *reinterpret_cast<const f32x4*>(sl + rr);
            f32x4 D4 = {};
            if (ROLE_DK) D4 = *reinterpret_cast<const f32x4*>(sl + kStage + rr);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * gg + e;
              float pv = __builtin_amdgcn_exp2f(fmaf(p[r], c, -L4[e]));
              if (masked && q0 + rr + e < ki) pv = 0.0f;
              if (ROLE_DK) p[r] = pv * fmaf(dp[r], sc_d, -D4[e]);  // dS
              else p[r] = pv;
            }
          }
          // dV^T += dO^T P, or dK^T += Q^T dS, over the fragment's two 16-query steps
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const u32x4 pf = pack_step<S>(p, st);
#pragma unroll
            for (int f = 0; f < FD; ++f) acc[f] = S::mfma32x32x16(tfr[st][f], pf, acc[f]);
          }
        }
      };
      if (a.causal && q0 < kw + 31) block(std::true_type{});
      else block(std::false_type{});
    }
    store_stage(smem + ((it + 1) & 1) * STG);
    __syncthreads();
  }

  // the second half's partial sums to the first, added in that order
  float* xbuf = reinterpret_cast<float*>(smem);
  if (hq == 1) half_put<FD>(xbuf, g, lane, acc, 0.0f, 0.0f);
  __syncthreads();
  if (hq == 1) return;
  {
    f32x16 a2[FD];
    float u0, u1;
    half_get<FD>(xbuf, g, lane, a2, u0, u1);
#pragma unroll
    for (int f = 0; f < FD; ++f) acc[f] += a2[f];
  }
  if (ki < a.s) {
    uint16_t* row = a.out + ((int64_t)b * a.s + ki) * a.ld3 + (int64_t)j * a.d + (ROLE_DK ? a.q : 2 * a.q);
#pragma unroll
    for (int f = 0; f < FD; ++f) store_t<S>(row, acc[f], 32 * f, a.d, h, 1.0f);
  }
}

// dQ: one workgroup per (pair z, 128 queries), the last (longest, when
// causal) query blocks first; wave w owns queries q0 + 32 (w % 4) + c and
// the key blocks of parity w / 4 (K and V tiles in LDS), recomputing p and
// dS in the transposed layout.
template <class S, int KS, int FD>
__global__ __launch_bounds__(kThreads) void flash_bwd_q_kernel(Args a) {
  constexpr int DK = 16 * KS, DV = 32 * FD;
  constexpr int KB = kStage * pitch<DV>(), STG = KB + kStage * pitch<DK>();
  static_assert(4 * 64 * (FD * 16 + 2) * 4 <= 2 * STG, "the halves' exchange fits in the stages");
  __shared__ __attribute__((aligned(16))) char smem[2 * STG];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, g = wave & 3, hk = wave >> 2;
  const int qb = a.nblk - 1 - (int)(blockIdx.x / a.Z), z = (int)(blockIdx.x % a.Z);
  const int b = z / a.heads, j = z % a.heads;
  const int64_t q0 = (int64_t)qb * kRows, qw = q0 + 32 * g, qi = qw + (lane & 31);
  const uint16_t* Qp = a.qkv + (int64_t)b * a.s * a.ld3 + (int64_t)j * a.d;
  const uint16_t* Kp = Qp + a.q;
  const uint16_t* Vp = Qp + 2 * a.q;
  const uint16_t* dOp = a.dO + (int64_t)b * a.s * a.ldo + (int64_t)j * a.d;
  const int64_t kv_end = a.causal ? min(a.s, q0 + kRows) : a.s;
  const int nit = (int)((kv_end + kStage - 1) / kStage);
  const int64_t wave_kend = qw >= a.s ? 0 : (a.causal ? min(kv_end, qw + 32) : kv_end);
  const float c = a.scale_log2, sc_d = a.scale;

  u32x4 qf[KS], df[KS];  // B operands of K Q^T and V dO^T: query qi, columns 16 ks + 8 h .. + 7
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int dd = 16 * ks + 8 * h;
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (qi < a.s && dd < a.d) {
      x = *reinterpret_cast<const u32x4*>(Qp + qi * a.ld3 + dd);
      y = *reinterpret_cast<const u32x4*>(dOp + qi * a.ldo + dd);
    }
    qf[ks] = x;
    df[ks] = y;
  }
  const float Lq = qi < a.s ? a.lse[(int64_t)z * a.s + qi] * kLog2e : 0.0f;
  const float Dq = qi < a.s ? a.D[(int64_t)z * a.s + qi] * sc_d : 0.0f;
  const int rowb = (int)(a.ld3 * 2);
  const auto krs = wave_rsrc(Kp, (a.s * a.ld3 - (int64_t)j * a.d - a.q) * 2);
  const auto vrs = wave_rsrc(Vp, (a.s * a.ld3 - (int64_t)j * a.d - 2 * a.q) * 2);
  TileCopy<kStage, DV> kt;
  TileCopy<kStage, DK> vt;
  kt.init(a.ld3, a.d, tid);
  vt.init(a.ld3, a.d, tid);
  f32x16 dq[FD];
#pragma unroll
  for (int f = 0; f < FD; ++f) dq[f] = f32x16{};

  if (nit > 0) {
    kt.load(krs, 0);
    vt.load(vrs, 0);
    kt.store(smem, tid);
    vt.store(smem + KB, tid);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // as in the forward: nothing in flight before the loop
  __syncthreads();
  for (int it = 0; it < nit; ++it) {
    // the next stage (past the end in the last iteration, as in the forward)
    kt.load(krs, (it + 1) * kStage * rowb);
    vt.load(vrs, (it + 1) * kStage * rowb);
    const int64_t k0 = (int64_t)it * kStage + hk * kBlk;  // this half's block
    if (k0 < wave_kend) {
      const char* sk = smem + (it & 1) * STG + hk * kBlk * pitch<DV>();
      const char* sv = smem + (it & 1) * STG + KB + hk * kBlk * pitch<DK>();
      // one 32-key fragment at a time (mf): x^T = K Q^T and dP^T = V dO^T,
      // rows (keys) k0 + 32 mf + frag_row(r, h), column query qi; the
      // fragment's LDS reads are all issued ahead of its products
      auto block = [&](auto masked) {
#pragma unroll
        for (int mf = 0; mf < 2; ++mf) {
          u32x4 kfr[KS], vfr[KS], tfr[2][FD];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            kfr[ks] = frag_rows<DV>(sk, 32 * mf, 16 * ks, lane);
            vfr[ks] = frag_rows<DK>(sv, 32 * mf, 16 * ks, lane);
          }
          f32x16 p = f32x16{}, dp = f32x16{};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            p = S::mfma32x32x16(kfr[ks], qf[ks], p);
            dp = S::mfma32x32x16(vfr[ks], df[ks], dp);
          }
          // (K^T read ahead only while its 8 FD registers fit beside the rest)
          constexpr bool kTAhead = FD <= 2;
          if constexpr (kTAhead) {
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
              for (int f = 0; f < FD; ++f) tfr[st][f] = frag_cols<DV>(sk, 32 * mf + 16 * st, 32 * f, lane);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float pv = __builtin_amdgcn_exp2f(fmaf(p[r], c, -Lq));
            if (masked) {
              const int64_t kk = k0 + 32 * mf + frag_row(r, h);
              if (kk >= a.s || (a.causal && kk > qi)) pv = 0.0f;
            }
            dp[r] = pv * fmaf(dp[r], sc_d, -Dq);  // dS^T
          }
          // dQ^T += K^T dS^T over the fragment's two 16-key steps
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const u32x4 sf = pack_step<S>(dp, st);
#pragma unroll
            for (int f = 0; f < FD; ++f)
              dq[f] = S::mfma32x32x16(kTAhead ? tfr[st][f] : frag_cols<DV>(sk, 32 * mf + 16 * st, 32 * f, lane), sf,
                                      dq[f]);
          }
        }
      };
      // keys past the end or after the query: last block and diagonal only (wave-uniform)
      if (k0 + kBlk > a.s || (a.causal && k0 + kBlk - 1 > qw)) block(std::true_type{});
      else block(std::false_type{});
    }
    {
      char* nx = smem + ((it + 1) & 1) * STG;
      kt.store(nx, tid);
      vt.store(nx + KB, tid);
    }
    __syncthreads();
  }

  // the second half's partial sums to the first, added in that order
  float* xbuf = reinterpret_cast<float*>(smem);
  if (hk == 1) half_put<FD>(xbuf, g, lane, dq, 0.0f, 0.0f);
  __syncthreads();
  if (hk == 1) return;
  {
    f32x16 d2[FD];
    float u0, u1;
    half_get<FD>(xbuf, g, lane, d2, u0, u1);
#pragma unroll
    for (int f = 0; f < FD; ++f) dq[f] += d2[f];
  }
  if (qi < a.s) {
    uint16_t* row = a.out + ((int64_t)b * a.s + qi) * a.ld3 + (int64_t)j * a.d;
#pragma unroll
    for (int f = 0; f < FD; ++f) store_t<S>(row, dq[f], 32 * f, a.d, h, 1.0f);
  }
}

// Launches for head width d <= 128: KS = ceil(d / 16) 16-wide steps of the
// d-sums, FD = ceil(d / 32) 32-row fragments of the d-wide results; the
// forward's column of ones where d is not a multiple of 32. Grid: nblk * Z
// workgroups.
#define TPMLP_FLASH_CASES(KERNEL, ...)                                                  \
  switch ((a.d + 15) / 16) {                                                            \
    case 1: hipLaunchKernelGGL((KERNEL<S, 1, 1 __VA_ARGS__>), grid, block, 0, st, a); break; \
    case 2: hipLaunchKernelGGL((KERNEL<S, 2, 1 __VA_ARGS__>), grid, block, 0, st, a); break; \
    case 3: hipLaunchKernelGGL((KERNEL<S, 3, 2 __VA_ARGS__>), grid, block, 0, st, a); break; \
    case 4: hipLaunchKernelGGL((KERNEL<S, 4, 2 __VA_ARGS__>), grid, block, 0, st, a); break; \
    case 5: hipLaunchKernelGGL((KERNEL<S, 5, 3 __VA_ARGS__>), grid, block, 0, st, a); break; \
    case 6: hipLaunchKernelGGL((KERNEL<S, 6, 3 __VA_ARGS__>), grid, block, 0, st, a); break; \
    case 7: hipLaunchKernelGGL((KERNEL<S, 7, 4 __VA_ARGS__>), grid, block, 0, st, a); break; \
    case 8: hipLaunchKernelGGL((KERNEL<S, 8, 4 __VA_ARGS__>), grid, block, 0, st, a); break; \
    default: return hipErrorInvalidValue;                                               \
  }

template <class S>
hipError_t launch_fwd(const Args& a, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)a.nblk * a.Z)), block(kThreads);
  if (a.d % 32) {
    TPMLP_FLASH_CASES(flash_fwd_kernel, , true)
  } else {
    TPMLP_FLASH_CASES(flash_fwd_kernel, , false)
  }
  return hipGetLastError();
}

template <class S>
hipError_t launch_bwd(const Args& a, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)a.nblk * a.Z)), block(kThreads);
  TPMLP_FLASH_CASES(flash_bwd_kv_kernel, , false)
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  TPMLP_FLASH_CASES(flash_bwd_kv_kernel, , true)
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  TPMLP_FLASH_CASES(flash_bwd_q_kernel)
  return hipGetLastError();
}
#undef TPMLP_FLASH_CASES

}  // namespace flash
}  // namespace tpmlp
