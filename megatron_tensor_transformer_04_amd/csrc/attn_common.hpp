// Pieces shared by the two attention-shard paths (tp_attn.hip, with the
// probabilities materialized; tp_attn_flash.hip, fused): shape and buffer
// checks, the derived sizes, and the row terms of the softmax backward.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "numerics.hpp"
#include "tp_attn.h"

namespace tpmlp {
namespace attn {

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t a256(size_t b) { return (b + 255) / 256 * 256; }

// Longest sequence of the materialized path: a softmax row of 4096 keys is
// 64 fp32 values per lane.
constexpr int64_t kMaxSeq = 4096;
// Widest head of the fused path: d <= 128 keeps a wave's accumulators of
// the d-wide results (up to 4 fragments of 32 x 32 per product) in registers.
constexpr int64_t kFlashMaxHeadDim = 128;

// Shape checks of both paths; `flash`: the fused path, which stores nothing
// of size seq x seq (no sequence cap) and needs head_dim <= 128.
inline int check_attn_shape(const tpattn_shape* s, bool flash) {
  if (!s) return TPMLP_ERR_NULL;
  if (s->dtype != TPMLP_F16 && s->dtype != TPMLP_BF16) return TPMLP_ERR_DTYPE;
  const int64_t lim = int64_t(1) << 30;
  const int64_t d[5] = {s->batch, s->seq, s->hidden, s->heads, s->head_dim};
  for (int64_t v : d)
    if (v <= 0 || v > lim) return TPMLP_ERR_SHAPE;
  const int64_t T = s->batch * s->seq, q = s->heads * s->head_dim;
  if (T > lim || q > lim / 3) return TPMLP_ERR_SHAPE;
  const int64_t pairs = s->batch * s->heads;
  if (pairs > 65535) return TPMLP_ERR_SHAPE;
  if (cdiv(T, 256) > 65535) return TPMLP_ERR_SHAPE;                  // grid y of the column-sum pass
  if (cdiv(T * s->heads, 256) > INT32_MAX) return TPMLP_ERR_SHAPE;  // row terms: one thread per (token, head)
  // tile counts of the projections' launches fit the 31-bit grid
  if (cdiv(T, 128) * cdiv(std::max<int64_t>(3 * q, s->hidden), 128) > INT32_MAX / 2 ||
      cdiv(s->hidden, 128) * cdiv(3 * q, 128) > INT32_MAX / 2)
    return TPMLP_ERR_SHAPE;
  if (flash) {
    if (s->head_dim > kFlashMaxHeadDim) return TPMLP_ERR_SHAPE;
    if (cdiv(s->seq, 128) * pairs > INT32_MAX) return TPMLP_ERR_SHAPE;  // one workgroup per (pair, 128 rows)
    // a sequence's QKV rows (and one block of rows past them) as one buffer range
    if ((s->seq + 128) * 3 * q * 2 >= (int64_t(1) << 31)) return TPMLP_ERR_SHAPE;
  } else {
    if ((double)pairs * (double)s->seq * (double)s->seq >= 1099511627776.0) return TPMLP_ERR_SHAPE;
    if (s->seq > kMaxSeq) return TPMLP_ERR_SHAPE;  // softmax rows are held in registers
    if (cdiv(s->seq, 128) * cdiv(s->seq, 128) > INT32_MAX / 2) return TPMLP_ERR_SHAPE;
  }
  if (s->seq % 8 || s->hidden % 8 || s->head_dim % 8) return TPMLP_ERR_ALIGN;
  return TPMLP_OK;
}

struct AttnDims {
  int64_t T, h, n, d, q, s, Z;
  float scale;
};

inline AttnDims dims(const tpattn_shape& sh) {
  AttnDims a;
  a.T = sh.batch * sh.seq;
  a.h = sh.hidden;
  a.n = sh.heads;
  a.d = sh.head_dim;
  a.q = sh.heads * sh.head_dim;
  a.s = sh.seq;
  a.Z = sh.batch * sh.heads;
  a.scale = (float)(1.0 / std::sqrt((double)sh.head_dim));
  return a;
}

struct Span2 {
  const void* p;
  size_t bytes;
};

inline bool overlaps(const Span2& a, const Span2& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Null, 16-byte alignment and overlap checks, in that order.
inline int check_spans(const Span2* in, int n_in, const Span2* out, int n_out) {
  for (int i = 0; i < n_in; ++i)
    if (!in[i].p) return TPMLP_ERR_NULL;
  for (int i = 0; i < n_out; ++i)
    if (!out[i].p) return TPMLP_ERR_NULL;
  for (int i = 0; i < n_in; ++i)
    if ((uintptr_t)in[i].p & 15u) return TPMLP_ERR_ALIGN;
  for (int i = 0; i < n_out; ++i)
    if ((uintptr_t)out[i].p & 15u) return TPMLP_ERR_ALIGN;
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlaps(out[i], in[j])) return TPMLP_ERR_ALIAS;
    for (int j = i + 1; j < n_out; ++j)
      if (overlaps(out[i], out[j])) return TPMLP_ERR_ALIAS;
  }
  return TPMLP_OK;
}

#define ATTN_HIP(expr)                              \
  do {                                              \
    if ((expr) != hipSuccess) return TPMLP_ERR_HIP; \
  } while (0)

// Row terms of the softmax backward: for each (sequence, head) pair z and
// query t, D[z][t] = sum_e dO[t][e] O[t][e] over the head's d columns (fp32,
// in e order). In exact arithmetic D = sum_k P[t][k] dP[t][k], since
// dP = dO V^T and O = P V; it is the term the softmax's backward subtracts.
// The loads of four 8-column chunks of each operand are issued before their
// products are added (in e order), so a thread has eight in flight.
template <class S>
__global__ __launch_bounds__(256) void softmax_rowdot_kernel(const typename S::T* __restrict__ dO,
                                                             const typename S::T* __restrict__ O, float* __restrict__ D,
                                                             int64_t T, int64_t s, int heads, int d, int64_t q) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // token * heads + head
  if (i >= T * heads) return;
  const int64_t t = i / heads;
  const int j = (int)(i % heads);
  const typename S::T* a = dO + t * q + (int64_t)j * d;
  const typename S::T* o = O + t * q + (int64_t)j * d;
  float acc = 0.0f;
  auto add = [&](const uint4& wa, const uint4& wo) {
    const uint32_t ua[4] = {wa.x, wa.y, wa.z, wa.w}, uo[4] = {wo.x, wo.y, wo.z, wo.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc += S::to_f((typename S::T)(ua[k] & 0xffffu)) * S::to_f((typename S::T)(uo[k] & 0xffffu));
      acc += S::to_f((typename S::T)(ua[k] >> 16)) * S::to_f((typename S::T)(uo[k] >> 16));
    }
  };
  int e = 0;
  for (; e + 32 <= d; e += 32) {
    uint4 wa[4], wo[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      wa[c] = *reinterpret_cast<const uint4*>(a + e + 8 * c);
      wo[c] = *reinterpret_cast<const uint4*>(o + e + 8 * c);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) add(wa[c], wo[c]);
  }
  for (; e < d; e += 8) add(*reinterpret_cast<const uint4*>(a + e), *reinterpret_cast<const uint4*>(o + e));
  const int64_t b = t / s, pos = t % s;
  D[((b * heads) + j) * s + pos] = acc;
}

}  // namespace attn
}  // namespace tpmlp
