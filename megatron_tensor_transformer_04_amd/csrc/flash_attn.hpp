// Fused attention core for gfx950: scores and probabilities never leave the
// chip. For one sequence b and head j, with Q, K, V the [seq, d] column
// blocks of QKV and x = Q K^T / sqrt(d) (keys after the query masked out
// when causal),
//   forward:  O = softmax(x) V and L = log sum_k exp(x_k) per query row,
//             one 64-key block at a time with a running maximum and sum per
//             row (the online form of the softmax);
//   backward: P = exp(x - L) recomputed from L, then
//             dV = P^T dO, dS = P (dO V^T - D) / sqrt(d), D = rowsum(dO O),
//             dK = dS^T Q (flash_bwd_kv_kernel, one workgroup per 128 keys)
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
// Lanes l and l + 32 hold the same row: the forward exchanges the running
// maximum between them once per key block and the running sums at the end.
#pragma once

#include <hip/hip_runtime.h>

#include "numerics.hpp"

namespace tpmlp {
namespace flash {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kThreads = 256;  // four waves, 32 rows each
constexpr int kRows = 128;     // rows (queries or keys) per workgroup
constexpr int kBlk = 64;       // keys (queries) per block of the inner loop

// Row pitch in bytes of a tile of C 16-bit columns in LDS: 16 bytes of
// padding put the 32 rows of a 16-byte fragment read, and the 4 rows of a
// transposing read, on distinct banks.
template <int C>
constexpr int pitch() {
  return C * 2 + 16;
}

// Rows [r0, r0 + R) and columns [0, C) of a row-major 16-bit matrix with row
// pitch ld, rows >= nrows and columns >= d read as 0, moved through
// registers into an LDS tile (register-staged so that the loads of the next
// block are in flight while the current one is computed).
template <int R, int C>
struct TileCopy {
  static constexpr int CH = C / 8, NCH = R * CH, N = (NCH + kThreads - 1) / kThreads;
  u32x4 v[N];
  __device__ __forceinline__ void load(const uint16_t* base, int64_t ld, int64_t r0, int64_t nrows, int d, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + i * kThreads, r = c / CH, cc = c % CH;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (c < NCH && r0 + r < nrows && cc * 8 < d) x = *reinterpret_cast<const u32x4*>(base + (r0 + r) * ld + cc * 8);
      v[i] = x;
    }
  }
  __device__ __forceinline__ void store(char* t, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + i * kThreads, r = c / CH, cc = c % CH;
      if (c < NCH) *reinterpret_cast<u32x4*>(t + r * pitch<C>() + cc * 16) = v[i];
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
    w[e] = (uint32_t)S::from_f(v[8 * st + 2 * e]) | ((uint32_t)S::from_f(v[8 * st + 2 * e + 1]) << 16);
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
      w[0] = (uint32_t)S::from_f(x[4 * g] * mul) | ((uint32_t)S::from_f(x[4 * g + 1] * mul) << 16);
      w[1] = (uint32_t)S::from_f(x[4 * g + 2] * mul) | ((uint32_t)S::from_f(x[4 * g + 3] * mul) << 16);
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
};

// Forward: one workgroup per (pair z, 128 queries), longest (last) query
// blocks first; wave w owns queries q0 + 32 w + c.
template <class S, int KS, int FD>
__global__ __launch_bounds__(kThreads) void flash_fwd_kernel(Args a) {
  constexpr int DK = 16 * KS, DV = 32 * FD;
  constexpr int KB = kBlk * pitch<DK>(), STG = KB + kBlk * pitch<DV>();
  __shared__ __attribute__((aligned(16))) char smem[2 * STG];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const int qb = a.nblk - 1 - (int)(blockIdx.x / a.Z), z = (int)(blockIdx.x % a.Z);
  const int b = z / a.heads, j = z % a.heads;
  const int64_t q0 = (int64_t)qb * kRows, qw = q0 + 32 * wave, qi = qw + (lane & 31);
  const uint16_t* Qp = a.qkv + (int64_t)b * a.s * a.ld3 + (int64_t)j * a.d;
  const uint16_t* Kp = Qp + a.q;
  const uint16_t* Vp = Qp + 2 * a.q;
  const int64_t kv_end = a.causal ? min(a.s, q0 + kRows) : a.s;
  const int nkb = (int)((kv_end + kBlk - 1) / kBlk);
  // keys this wave reads: none if all its queries are past the end, else up
  // to its last query when causal (wave-uniform)
  const int64_t wave_kend = qw >= a.s ? 0 : (a.causal ? min(kv_end, qw + 32) : kv_end);

  u32x4 qf[KS];  // B operand of K Q^T: query qi, columns 16 ks + 8 h .. + 7
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int dd = 16 * ks + 8 * h;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (qi < a.s && dd < a.d) v = *reinterpret_cast<const u32x4*>(Qp + qi * a.ld3 + dd);
    qf[ks] = v;
  }
  TileCopy<kBlk, DK> kt;
  TileCopy<kBlk, DV> vt;
  f32x16 o[FD];
#pragma unroll
  for (int f = 0; f < FD; ++f) o[f] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;

  if (nkb > 0) {
    kt.load(Kp, a.ld3, 0, a.s, a.d, tid);
    vt.load(Vp, a.ld3, 0, a.s, a.d, tid);
    kt.store(smem, tid);
    vt.store(smem + KB, tid);
  }
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int64_t k0 = (int64_t)kb * kBlk;
    if (kb + 1 < nkb) {
      kt.load(Kp, a.ld3, k0 + kBlk, a.s, a.d, tid);
      vt.load(Vp, a.ld3, k0 + kBlk, a.s, a.d, tid);
    }
    if (k0 < wave_kend) {
      const char* sk = smem + (kb & 1) * STG;
      const char* sv = sk + KB;
      // x^T = K Q^T, scaled to log2 units: keys k0 + 32 mf + frag_row(r, h)
      f32x16 sc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mf = 0; mf < 2; ++mf)
          sc[mf] = S::mfma32x32x16(frag_rows<DK>(sk, 32 * mf, 16 * ks, lane), qf[ks], sc[mf]);
      const bool diag = a.causal && k0 + kBlk - 1 > qw;
      float mb = -INFINITY;
#pragma unroll
      for (int mf = 0; mf < 2; ++mf)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t ki = k0 + 32 * mf + frag_row(r, h);
          float v = sc[mf][r] * a.scale_log2;
          if (ki >= a.s || (diag && ki > qi)) v = -INFINITY;
          sc[mf][r] = v;
          mb = fmaxf(mb, v);
        }
      mb = fmaxf(mb, __shfl_xor(mb, 32));
      const float m_new = fmaxf(m_run, mb);
      // while no key of the row has been seen (m_new = -inf) every p is 0 and
      // the state stays as it is
      const float msub = m_new == -INFINITY ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - msub);
      float ls = 0.0f;
#pragma unroll
      for (int mf = 0; mf < 2; ++mf)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(sc[mf][r] - msub);
          sc[mf][r] = p;
          ls += p;
        }
      l_run = l_run * alpha + ls;
      m_run = m_new;
#pragma unroll
      for (int f = 0; f < FD; ++f) o[f] *= alpha;
      // O^T += V^T P^T over four 16-key steps
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const u32x4 pf = pack_step<S>(sc[st >> 1], st & 1);
#pragma unroll
        for (int f = 0; f < FD; ++f) o[f] = S::mfma32x32x16(frag_cols<DV>(sv, 16 * st, 32 * f, lane), pf, o[f]);
      }
    }
    // the other stage was last read in the previous iteration, before the
    // barrier that ended it
    if (kb + 1 < nkb) {
      char* nx = smem + ((kb + 1) & 1) * STG;
      kt.store(nx, tid);
      vt.store(nx + KB, tid);
    }
    __syncthreads();
  }

  // O = O^T / l (rows d < a.d); L = (m + log2 l) ln 2
  const float l_all = l_run + __shfl_xor(l_run, 32);
  if (qi < a.s) {
    const float inv = 1.0f / l_all;
    uint16_t* orow = a.out + ((int64_t)b * a.s + qi) * a.ldo + (int64_t)j * a.d;
#pragma unroll
    for (int f = 0; f < FD; ++f) store_t<S>(orow, o[f], 32 * f, a.d, h, inv);
    if (h == 0) a.lse[(int64_t)z * a.s + qi] = (m_run + log2f(l_all)) * kLn2;
  }
}

// dK and dV: one workgroup per (pair z, 128 keys), first (longest, when
// causal) key blocks first; wave w owns keys k0 + 32 w + c and loops over
// 64-query blocks (Q and dO tiles, L and D of those queries in LDS).
template <class S, int KS, int FD>
__global__ __launch_bounds__(kThreads) void flash_bwd_kv_kernel(Args a) {
  constexpr int DV = 32 * FD;
  constexpr int TB = kBlk * pitch<DV>(), STG = 2 * TB + 2 * kBlk * 4;
  __shared__ __attribute__((aligned(16))) char smem[2 * STG];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const int kblk = (int)(blockIdx.x / a.Z), z = (int)(blockIdx.x % a.Z);
  const int b = z / a.heads, j = z % a.heads;
  const int64_t k0 = (int64_t)kblk * kRows, kw = k0 + 32 * wave, ki = kw + (lane & 31);
  const uint16_t* Qp = a.qkv + (int64_t)b * a.s * a.ld3 + (int64_t)j * a.d;
  const uint16_t* Kp = Qp + a.q;
  const uint16_t* Vp = Qp + 2 * a.q;
  const uint16_t* dOp = a.dO + (int64_t)b * a.s * a.ldo + (int64_t)j * a.d;
  const float* Lz = a.lse + (int64_t)z * a.s;
  const float* Dz = a.D + (int64_t)z * a.s;
  const int64_t qstart = a.causal ? k0 : 0;  // queries before the block's first key see none of its keys
  const int nqb = (int)((a.s - qstart + kBlk - 1) / kBlk);
  const bool live = kw < a.s;

  u32x4 kf[KS], vf[KS];  // B operands of Q K^T and dO V^T: key ki, columns 16 ks + 8 h .. + 7
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int dd = 16 * ks + 8 * h;
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (ki < a.s && dd < a.d) {
      x = *reinterpret_cast<const u32x4*>(Kp + ki * a.ld3 + dd);
      y = *reinterpret_cast<const u32x4*>(Vp + ki * a.ld3 + dd);
    }
    kf[ks] = x;
    vf[ks] = y;
  }
  TileCopy<kBlk, DV> qt, dt;
  float rowv = 0.0f;  // thread t < 64: L (log2 units) of query t of the block; 64 <= t < 128: D
  auto load_rows = [&](int64_t r0) {
    const int t = tid & 63;
    if (tid < 64) rowv = r0 + t < a.s ? Lz[r0 + t] * kLog2e : INFINITY;  // P = 0 past the end
    else if (tid < 128) rowv = r0 + t < a.s ? Dz[r0 + t] : 0.0f;
  };
  auto store_stage = [&](char* t) {
    qt.store(t, tid);
    dt.store(t + TB, tid);
    if (tid < 128) reinterpret_cast<float*>(t + 2 * TB)[tid] = rowv;
  };
  f32x16 dk[FD], dv[FD];
#pragma unroll
  for (int f = 0; f < FD; ++f) dk[f] = dv[f] = f32x16{};

  if (nqb > 0) {
    qt.load(Qp, a.ld3, qstart, a.s, a.d, tid);
    dt.load(dOp, a.ldo, qstart, a.s, a.d, tid);
    load_rows(qstart);
    store_stage(smem);
  }
  __syncthreads();
  for (int ib = 0; ib < nqb; ++ib) {
    const int64_t q0 = qstart + (int64_t)ib * kBlk;
    if (ib + 1 < nqb) {
      qt.load(Qp, a.ld3, q0 + kBlk, a.s, a.d, tid);
      dt.load(dOp, a.ldo, q0 + kBlk, a.s, a.d, tid);
      load_rows(q0 + kBlk);
    }
    // causal: a block whose queries all precede the wave's keys has P = 0
    if (live && !(a.causal && q0 + kBlk - 1 < kw)) {
      const char* sq = smem + (ib & 1) * STG;
      const char* sd = sq + TB;
      const float* sl = reinterpret_cast<const float*>(sq + 2 * TB);
      // x = Q K^T and dP = dO V^T: rows (queries) q0 + 32 mf + frag_row(r, h), column key ki
      f32x16 p[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mf = 0; mf < 2; ++mf) {
          p[mf] = S::mfma32x32x16(frag_rows<DV>(sq, 32 * mf, 16 * ks, lane), kf[ks], p[mf]);
          dp[mf] = S::mfma32x32x16(frag_rows<DV>(sd, 32 * mf, 16 * ks, lane), vf[ks], dp[mf]);
        }
      const bool diag = a.causal && q0 < kw + 31;
#pragma unroll
      for (int mf = 0; mf < 2; ++mf)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int rr = 32 * mf + 8 * g + 4 * h;
          const f32x4 L4 = *reinterpret_cast<const f32x4*>(sl + rr);
          const f32x4 D4 = *reinterpret_cast<const f32x4*>(sl + kBlk + rr);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            float pv = __builtin_amdgcn_exp2f(p[mf][r] * a.scale_log2 - L4[e]);
            if (diag && q0 + rr + e < ki) pv = 0.0f;
            p[mf][r] = pv;
            dp[mf][r] = pv * (dp[mf][r] - D4[e]) * a.scale;  // dS
          }
        }
      // dV^T += dO^T P and dK^T += Q^T dS over four 16-query steps
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const u32x4 pf = pack_step<S>(p[st >> 1], st & 1);
        const u32x4 sf = pack_step<S>(dp[st >> 1], st & 1);
#pragma unroll
        for (int f = 0; f < FD; ++f) {
          dv[f] = S::mfma32x32x16(frag_cols<DV>(sd, 16 * st, 32 * f, lane), pf, dv[f]);
          dk[f] = S::mfma32x32x16(frag_cols<DV>(sq, 16 * st, 32 * f, lane), sf, dk[f]);
        }
      }
    }
    if (ib + 1 < nqb) store_stage(smem + ((ib + 1) & 1) * STG);
    __syncthreads();
  }

  if (ki < a.s) {
    uint16_t* row = a.out + ((int64_t)b * a.s + ki) * a.ld3 + (int64_t)j * a.d;
#pragma unroll
    for (int f = 0; f < FD; ++f) {
      store_t<S>(row + a.q, dk[f], 32 * f, a.d, h, 1.0f);
      store_t<S>(row + 2 * a.q, dv[f], 32 * f, a.d, h, 1.0f);
    }
  }
}

// dQ: one workgroup per (pair z, 128 queries), longest query blocks first;
// wave w owns queries q0 + 32 w + c and loops over 64-key blocks (K and V
// tiles in LDS), recomputing P^T and dS^T in the transposed layout.
template <class S, int KS, int FD>
__global__ __launch_bounds__(kThreads) void flash_bwd_q_kernel(Args a) {
  constexpr int DK = 16 * KS, DV = 32 * FD;
  constexpr int KB = kBlk * pitch<DV>(), STG = KB + kBlk * pitch<DK>();
  __shared__ __attribute__((aligned(16))) char smem[2 * STG];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const int qb = a.nblk - 1 - (int)(blockIdx.x / a.Z), z = (int)(blockIdx.x % a.Z);
  const int b = z / a.heads, j = z % a.heads;
  const int64_t q0 = (int64_t)qb * kRows, qw = q0 + 32 * wave, qi = qw + (lane & 31);
  const uint16_t* Qp = a.qkv + (int64_t)b * a.s * a.ld3 + (int64_t)j * a.d;
  const uint16_t* Kp = Qp + a.q;
  const uint16_t* Vp = Qp + 2 * a.q;
  const uint16_t* dOp = a.dO + (int64_t)b * a.s * a.ldo + (int64_t)j * a.d;
  const int64_t kv_end = a.causal ? min(a.s, q0 + kRows) : a.s;
  const int nkb = (int)((kv_end + kBlk - 1) / kBlk);
  const int64_t wave_kend = qw >= a.s ? 0 : (a.causal ? min(kv_end, qw + 32) : kv_end);

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
  const float Dq = qi < a.s ? a.D[(int64_t)z * a.s + qi] : 0.0f;
  TileCopy<kBlk, DV> kt;
  TileCopy<kBlk, DK> vt;
  f32x16 dq[FD];
#pragma unroll
  for (int f = 0; f < FD; ++f) dq[f] = f32x16{};

  if (nkb > 0) {
    kt.load(Kp, a.ld3, 0, a.s, a.d, tid);
    vt.load(Vp, a.ld3, 0, a.s, a.d, tid);
    kt.store(smem, tid);
    vt.store(smem + KB, tid);
  }
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int64_t k0 = (int64_t)kb * kBlk;
    if (kb + 1 < nkb) {
      kt.load(Kp, a.ld3, k0 + kBlk, a.s, a.d, tid);
      vt.load(Vp, a.ld3, k0 + kBlk, a.s, a.d, tid);
    }
    if (k0 < wave_kend) {
      const char* sk = smem + (kb & 1) * STG;
      const char* sv = sk + KB;
      // x^T = K Q^T and dP^T = V dO^T: rows (keys) k0 + 32 mf + frag_row(r, h), column query qi
      f32x16 p[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mf = 0; mf < 2; ++mf) {
          p[mf] = S::mfma32x32x16(frag_rows<DV>(sk, 32 * mf, 16 * ks, lane), qf[ks], p[mf]);
          dp[mf] = S::mfma32x32x16(frag_rows<DK>(sv, 32 * mf, 16 * ks, lane), df[ks], dp[mf]);
        }
      const bool diag = a.causal && k0 + kBlk - 1 > qw;
#pragma unroll
      for (int mf = 0; mf < 2; ++mf)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t kk = k0 + 32 * mf + frag_row(r, h);
          float pv = __builtin_amdgcn_exp2f(p[mf][r] * a.scale_log2 - Lq);
          if (kk >= a.s || (diag && kk > qi)) pv = 0.0f;
          dp[mf][r] = pv * (dp[mf][r] - Dq) * a.scale;  // dS^T
        }
      // dQ^T += K^T dS^T over four 16-key steps
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const u32x4 sf = pack_step<S>(dp[st >> 1], st & 1);
#pragma unroll
        for (int f = 0; f < FD; ++f) dq[f] = S::mfma32x32x16(frag_cols<DV>(sk, 16 * st, 32 * f, lane), sf, dq[f]);
      }
    }
    if (kb + 1 < nkb) {
      char* nx = smem + ((kb + 1) & 1) * STG;
      kt.store(nx, tid);
      vt.store(nx + KB, tid);
    }
    __syncthreads();
  }

  if (qi < a.s) {
    uint16_t* row = a.out + ((int64_t)b * a.s + qi) * a.ld3 + (int64_t)j * a.d;
#pragma unroll
    for (int f = 0; f < FD; ++f) store_t<S>(row, dq[f], 32 * f, a.d, h, 1.0f);
  }
}

// Launch one of the three kernels for head width d <= 128: KS = ceil(d / 16)
// 16-wide steps of the d-sums, FD = ceil(d / 32) 32-row fragments of the
// d-wide results. Grid: nblk * Z workgroups.
#define TPMLP_FLASH_LAUNCH(KERNEL)                                                  \
  template <class S>                                                               \
  hipError_t launch_##KERNEL(const Args& a, hipStream_t st) {                      \
    const dim3 grid((unsigned)((int64_t)a.nblk * a.Z)), block(kThreads);           \
    switch ((a.d + 15) / 16) {                                                     \
      case 1: hipLaunchKernelGGL((KERNEL<S, 1, 1>), grid, block, 0, st, a); break; \
      case 2: hipLaunchKernelGGL((KERNEL<S, 2, 1>), grid, block, 0, st, a); break; \
      case 3: hipLaunchKernelGGL((KERNEL<S, 3, 2>), grid, block, 0, st, a); break; \
      case 4: hipLaunchKernelGGL((KERNEL<S, 4, 2>), grid, block, 0, st, a); break; \
      case 5: hipLaunchKernelGGL((KERNEL<S, 5, 3>), grid, block, 0, st, a); break; \
      case 6: hipLaunchKernelGGL((KERNEL<S, 6, 3>), grid, block, 0, st, a); break; \
      case 7: hipLaunchKernelGGL((KERNEL<S, 7, 4>), grid, block, 0, st, a); break; \
      case 8: hipLaunchKernelGGL((KERNEL<S, 8, 4>), grid, block, 0, st, a); break; \
      default: return hipErrorInvalidValue;                                        \
    }                                                                              \
    return hipGetLastError();                                                      \
  }

TPMLP_FLASH_LAUNCH(flash_fwd_kernel)
TPMLP_FLASH_LAUNCH(flash_bwd_kv_kernel)
TPMLP_FLASH_LAUNCH(flash_bwd_q_kernel)
#undef TPMLP_FLASH_LAUNCH

}  // namespace flash
}  // namespace tpmlp
