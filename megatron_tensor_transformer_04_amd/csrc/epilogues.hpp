// GEMM epilogues: what happens to each fp32 accumulator C[m][n] of a tile.
//
// Every epilogue exposes
//   float apply(int64_t m, int64_t n, float acc)   store the result, return
//                                                  the value that enters the
//                                                  optional column sum;
//   static constexpr bool kColSum                  whether the kernel also
//                                                  reduces the tile's columns;
//   void colsum(int tile_m, int64_t n, float s)    store one tile's sum.
// apply() is only called for in-range (m, n).
//
// For the tile-wise epilogue of the direct-to-LDS engine (which loads and
// stores whole 16-byte row chunks) every epilogue also exposes
//   static constexpr int kOuts                     16-bit outputs (1 or 2);
//   static constexpr bool kInput                   whether it reads a [M][N]
//                                                  16-bit input at (m, n);
//   const T* input() / T* output(k) / int64_t ld   those tensors (an output
//                                                  may be null: not kept);
//   float colparam(int64_t n)                      a per-column value;
//   static constexpr bool kColParam                whether it has one other
//                                                  than 0, and then
//   const T* colvec()                              the 16-bit vector it is
//                                                  read from (colparam(n) =
//                                                  colvec()[n]);
//   float eval(float acc, float colp, float in, float (&o)[2])
//                                                  the fp32 outputs before
//                                                  rounding, and the value
//                                                  that enters the column sum.
#pragma once

#include "numerics.hpp"

namespace tpmlp {

// C = round(acc): the row-parallel partial Yp, dB, dA and dXp.
template <class S>
struct EpiStore {
  typename S::T* out;
  int64_t ld;
  static constexpr bool kColSum = false;
  static constexpr int kOuts = 1;
  static constexpr bool kInput = false;
  static constexpr bool kTailSplit = true;  // a plain store: k-split tail tiles may finish it elsewhere
  static constexpr bool kDirectF32 = false;
  static constexpr bool kColParam = false;
  __device__ __forceinline__ const typename S::T* input() const { return nullptr; }
  __device__ __forceinline__ typename S::T* output(int) const { return out; }
  __device__ __forceinline__ float colparam(int64_t) const { return 0.0f; }
  __device__ __forceinline__ const typename S::T* colvec() const { return nullptr; }
  __device__ __forceinline__ float eval(float acc, float, float, float (&o)[2]) const {
    o[0] = acc;
    return 0.0f;
  }
  __device__ __forceinline__ float apply(int64_t m, int64_t n, float acc) const {
    out[m * ld + n] = S::from_f(acc);
    return 0.0f;
  }
  __device__ __forceinline__ void colsum(int, int64_t, float) const {}
};

// Fused bias + GeLU after the column-parallel GEMM:
//   z = acc + b1[n];  Z[m][n] = round(z);  H[m][n] = round(gelu(z)).
// Both outputs come from the one fp32 value z ("Training GPT-2 with
// Megatron-LM", section 6.2, fused_bias_gelu).
template <class S>
struct EpiBiasGelu {
  const typename S::T* bias;
  typename S::T* z;
  typename S::T* h;  // may be null: H not kept
  int64_t ld;
  static constexpr bool kColSum = false;
  static constexpr int kOuts = 2;
  static constexpr bool kInput = false;
  static constexpr bool kTailSplit = false;
  static constexpr bool kDirectF32 = false;
  static constexpr bool kColParam = true;
  __device__ __forceinline__ const typename S::T* input() const { return nullptr; }
  __device__ __forceinline__ typename S::T* output(int k) const { return k ? h : z; }
  __device__ __forceinline__ float colparam(int64_t n) const { return S::to_f(bias[n]); }
  __device__ __forceinline__ const typename S::T* colvec() const { return bias; }
  __device__ __forceinline__ float eval(float acc, float colp, float, float (&o)[2]) const {
    const float v = acc + colp;
    o[0] = v;
    o[1] = gelu_tanh(v);
    return 0.0f;
  }
  __device__ __forceinline__ float apply(int64_t m, int64_t n, float acc) const {
    const float v = acc + S::to_f(bias[n]);
    z[m * ld + n] = S::from_f(v);
    if (h) h[m * ld + n] = S::from_f(gelu_tanh(v));
    return 0.0f;
  }
  __device__ __forceinline__ void colsum(int, int64_t, float) const {}
};

// Backward through the GeLU after the dH GEMM (dH = dY B_i^T):
//   d = acc * gelu'(Z[m][n]);  dZ[m][n] = round(d);
// and the fp32 column sums of d over the tile's rows, the per-tile partials
// of db1 = sum over tokens of dZ.
template <class S>
struct EpiGeluGrad {
  const typename S::T* zin;
  typename S::T* dz;
  float* partial;  // [tiles_m][ld]
  int64_t ld;
  // read Z with non-temporal loads (the direct-load engine's epilogue): set
  // for a Z at least as large as the MALL, which it streams through once
  // (measured on MI355X: 16384 x 10240, 2.64 -> 2.59 ms; for 8192 x 2560,
  // which the MALL can still hold from the forward, such loads were slower)
  bool stream = false;
  static constexpr bool kColSum = true;
  static constexpr int kOuts = 1;
  static constexpr bool kInput = true;
  static constexpr bool kTailSplit = false;
  static constexpr bool kDirectF32 = false;
  static constexpr bool kColParam = false;
  __device__ __forceinline__ const typename S::T* input() const { return zin; }
  __device__ __forceinline__ typename S::T* output(int) const { return dz; }
  __device__ __forceinline__ float colparam(int64_t) const { return 0.0f; }
  __device__ __forceinline__ const typename S::T* colvec() const { return nullptr; }
  __device__ __forceinline__ float eval(float acc, float, float zv, float (&o)[2]) const {
    const float d = acc * gelu_tanh_grad(zv);
    o[0] = d;
    return d;
  }
  __device__ __forceinline__ float apply(int64_t m, int64_t n, float acc) const {
    const float d = acc * gelu_tanh_grad(S::to_f(zin[m * ld + n]));
    dz[m * ld + n] = S::from_f(d);
    return d;
  }
  __device__ __forceinline__ void colsum(int tile_m, int64_t n, float s) const {
    partial[(int64_t)tile_m * ld + n] = s;
  }
};

// Gradient accumulation into fp32 main gradients (beta = 1): the weight
// gradient of this micro-batch is added to an fp32 buffer that the caller
// keeps across micro-batches, main[m][n] += acc, without an intermediate
// rounding to the storage dtype. The pages train with fp16 products and fp32
// master weights ("Megatron-LM overview", section 3.1) and accumulate
// gradients over micro-batches ("Training GPT-2 with Megatron-LM",
// section 4.3, --gradient-accumulation-steps). kDirectF32: the
// direct-to-LDS engine reads and writes the fp32 rows straight from its
// accumulators (no 16-bit staging).
template <class S>
struct EpiAccumF32 {
  float* main;
  int64_t ld;
  static constexpr bool kColSum = false;
  static constexpr int kOuts = 1;
  static constexpr bool kInput = false;
  static constexpr bool kTailSplit = false;
  static constexpr bool kDirectF32 = true;
  static constexpr bool kColParam = false;
  __device__ __forceinline__ const typename S::T* input() const { return nullptr; }
  __device__ __forceinline__ typename S::T* output(int) const { return nullptr; }
  __device__ __forceinline__ float colparam(int64_t) const { return 0.0f; }
  __device__ __forceinline__ const typename S::T* colvec() const { return nullptr; }
  __device__ __forceinline__ float eval(float acc, float, float, float (&o)[2]) const {
    o[0] = acc;
    return 0.0f;
  }
  __device__ __forceinline__ float apply(int64_t m, int64_t n, float acc) const {
    main[m * ld + n] += acc;
    return 0.0f;
  }
  __device__ __forceinline__ void colsum(int, int64_t, float) const {}
};

// Any per-element epilogue, with C stored transposed: C[m][n] goes where the
// inner epilogue puts element (n, m). For the register-staged and fp32
// engines (per-element apply); used where an operand needs the GeLU on load
// but sits on the Q side of the GEMM that produces the wanted orientation.
template <class Inner>
struct EpiTransposed {
  Inner inner;
  static_assert(!Inner::kColSum, "column sums of a transposed store are row sums");
  static constexpr bool kColSum = false;
  static constexpr int kOuts = 1;
  static constexpr bool kInput = false;
  static constexpr bool kTailSplit = false;
  static constexpr bool kDirectF32 = false;
  static constexpr bool kColParam = false;
  __device__ __forceinline__ float apply(int64_t m, int64_t n, float acc) const { return inner.apply(n, m, acc); }
  __device__ __forceinline__ void colsum(int, int64_t, float) const {}
};

}  // namespace tpmlp
