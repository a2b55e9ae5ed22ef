// Storage formats, fp32 <-> 16-bit conversions and the tanh-GeLU for gfx950.
//
// GeLU is the tanh approximation of Hendrycks & Gimpel, "Gaussian Error
// Linear Units" (2016); the pages fuse it with the first linear's bias
// ("Training GPT-2 with Megatron-LM", section 6.2, fused_bias_gelu) without
// stating a formula. tanh(u) enters only through (1 + tanh(u)) / 2, the
// logistic function of 2u, see gelu_sigma.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// fp32 storage (the plain-FMA path)
struct StoreF32 {
  using T = float;
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float v) { return v; }
};

// IEEE binary16 storage; the hardware conversion rounds to nearest-even.
struct StoreF16 {
  using T = uint16_t;
  static __device__ __forceinline__ float to_f(uint16_t v) {
    return (float)__builtin_bit_cast(_Float16, v);
  }
  static __device__ __forceinline__ uint16_t from_f(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
  }
  // a and b rounded (as from_f) into the low and high halves: one v_cvt_pk_f16_f32
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
  }
  static __device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

// bfloat16 storage: the top 16 bits of an fp32. fp32 -> bf16 is gfx950's
// v_cvt_pk_bf16_f32, which rounds to nearest-even (NaN stays NaN).
struct StoreBF16 {
  using T = uint16_t;
  static __device__ __forceinline__ float to_f(uint16_t v) {
    return __builtin_bit_cast(float, (uint32_t)v << 16);
  }
  static __device__ __forceinline__ uint16_t from_f(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
  }
  // a and b rounded (as from_f) into the low and high halves: one v_cvt_pk_bf16_f32
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
  }
  static __device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

constexpr float kSqrt2OverPi = 0.7978845608028654f;
constexpr float kGeluC = 0.044715f;

// With u = sqrt(2/pi) (x + c x^3) and t = tanh(u), (1 + t) / 2 is the
// logistic function of 2u:
//   s = (1 + t) / 2 = 1 / (1 + exp(-2u)) = 1 / (1 + 2^(-x (A + B x^2))),
//   A = 2 sqrt(2/pi) log2(e),  B = A c,
// so gelu(x) = x (1 + t) / 2 = x s, and, since ds/du = 2 s (1 - s),
//   gelu'(x) = s + x s (1 - s) 2 sqrt(2/pi) (1 + 3 c x^2)
//            = s (1 + (1 - s) x (K1 + K2 x^2)),  K1 = 2 sqrt(2/pi), K2 = 3 c K1.
// One exp2 and one reciprocal per element and no clamp: for large -x the
// power overflows to +inf and s = 1/inf = 0; for large +x it underflows to
// 0 and s = 1.
constexpr float kGeluA = 2.0f * kSqrt2OverPi * 1.4426950408889634f;
constexpr float kGeluB = kGeluA * kGeluC;
constexpr float kGeluK1 = 2.0f * kSqrt2OverPi;
constexpr float kGeluK2 = 3.0f * kGeluC * kGeluK1;

__device__ __forceinline__ float gelu_sigma(float x, float x2) {
  const float p = -x * fmaf(kGeluB, x2, kGeluA);
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(p));
}

// gelu(x) = x s
__device__ __forceinline__ float gelu_tanh(float x) { return x * gelu_sigma(x, x * x); }

// gelu'(x) = s (1 + (1 - s) q), q = x (K1 + K2 x^2). x is clamped to
// [-16, 16] inside q only: beyond it s is exactly 0 or 1 in fp32 (the power
// is 2^(+-458) or further), so (1 - s) q or s (...) is exactly 0 there and
// the clamp changes nothing but keeps q finite.
__device__ __forceinline__ float gelu_tanh_grad(float x) {
  const float s = gelu_sigma(x, x * x);
  const float xc = __builtin_amdgcn_fmed3f(x, -16.0f, 16.0f);
  const float q = xc * fmaf(kGeluK2, xc * xc, kGeluK1);
  return s * fmaf(1.0f - s, q, 1.0f);
}

// Apply gelu to the eight 16-bit values packed in one 16-byte chunk.
template <class S>
__device__ __forceinline__ u32x4 gelu_chunk(u32x4 v) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint16_t lo = (uint16_t)(v[w] & 0xffffu), hi = (uint16_t)(v[w] >> 16);
    const uint16_t glo = S::from_f(gelu_tanh(S::to_f(lo)));
    const uint16_t ghi = S::from_f(gelu_tanh(S::to_f(hi)));
    r[w] = (uint32_t)glo | ((uint32_t)ghi << 16);
  }
  return r;
}

}  // namespace tpmlp
