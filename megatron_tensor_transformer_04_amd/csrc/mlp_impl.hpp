// Launch sequences of the tensor-parallel MLP shard: the forward (F1: X A_i
// with fused bias + GeLU, F2: H_i B_i), the backward (B1: dY B_i^T with fused
// gelu' and db1 column partials, B5: db1 finish, B2: H_i^T dY, B3: X^T dZ_i,
// B4: dZ_i A_i^T), the recomputation of Z for the selective-recompute
// backward, and the planned GEMMs the attention shard uses. Instantiated
// once per storage type, each in its own translation unit (mlp_f32.hip,
// mlp_f16.hip, mlp_bf16.hip), so that the three compile in parallel; the C
// ABI (tp_mlp.hip) sees them through TPMLP_MLP_INSTANCES(extern, ...).
#pragma once

#include "mlp_plan.hpp"

namespace tpmlp {

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
// xs: X held as row slices (sequence parallelism), or NULL for the dense X.
int fwd_impl(const tpmlp_shape& s, const void* X, const void* A, const void* b1, const void* B, void* Z, void* H,
             void* Yp, void* ws, size_t ws_bytes, hipStream_t st, void* const* ev, const RowSlices* xs = nullptr) {
  using T = typename S::T;
  const int64_t Tn = s.tokens, h = s.hidden, f = s.ffn_shard;
  const FwdWs w = fwd_ws(s);
  const bool room = ws && ws_bytes >= w.total;
  char* wsb = static_cast<char*>(ws);
  TPMLP_TRY(record(ev, 0, st));
  // TA + F1: Z = X A_i + b1 (and H = gelu(Z)); P = X [T,h] k-contiguous,
  // Q = A_i [h,f] (n-contiguous), or its transpose A_i^T [f,h] (k-contiguous)
  // With TPMLP_LAYOUT_WEIGHTS_STAGED the copies of A_i and B_i are already in
  // the workspace (written by an earlier call from the same weights).
  const bool have_copies = weights_staged(s);
  if (room && w.at) {
    if (!have_copies) TPMLP_HIP((run_transpose<S, false>(A, wsb + w.at_off, h, f, st)));
    TPMLP_TRY(record(ev, 1, st));
    const EpiBiasGelu<S> epi{(const T*)b1, (T*)Z, (T*)H, f};
    if (xs)
      TPMLP_HIP((run_gemm_sliced<S, true>(s.dtype, Tn, f, h, *xs, h, wsb + w.at_off, staged_ld(h), epi, st)));
    else
      TPMLP_HIP((run_gemm<S, true, true, false>(s.dtype, Tn, f, h, X, h, wsb + w.at_off, staged_ld(h), epi, st)));
  } else {
    TPMLP_TRY(record(ev, 1, st));
    const EpiBiasGelu<S> epi{(const T*)b1, (T*)Z, (T*)H, f};
    if (xs)
      TPMLP_HIP((run_gemm_sliced<S, false>(s.dtype, Tn, f, h, *xs, h, A, f, epi, st)));
    else
      TPMLP_HIP((run_gemm<S, true, false, false>(s.dtype, Tn, f, h, X, h, A, f, epi, st)));
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
    if (!have_copies) TPMLP_HIP((run_transpose<S, false>(B, wsb + w.bt_off, f, h, st)));
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

  // Z streams through B1's epilogue once; from the MALL's 256 MiB on it is
  // read with non-temporal loads
  const EpiGeluGrad<S> epi_b1{(const T*)Z, (T*)dZ, part, f, Tn * f * (int64_t)sizeof(T) >= (int64_t(256) << 20)};

  TPMLP_TRY(record(ev, 0, st));
  // B1: dZ = (dY B_i^T) * gelu'(Z), plus per-tile column sums; Q[k][n] = B_i[n][k] is k-contiguous.
  // With B_i^T [h,f] given, Q[k][n] = B_i^T[k][n] is n-contiguous: it is read
  // in place, or from a k-contiguous copy B_i [f][h + pad] staged first.
  if (!bt) {
    TPMLP_HIP((run_gemm<S, true, true, false>(s.dtype, Tn, f, h, dY, h, B, h, epi_b1, st)));
  } else if (room && w.stage_b1) {
    TPMLP_HIP((run_transpose<S, false>(B, wsb + w.bs_off, h, f, st)));
    TPMLP_HIP((run_gemm<S, true, true, false>(s.dtype, Tn, f, h, dY, h, wsb + w.bs_off, staged_ld(h), epi_b1, st)));
  } else {
    TPMLP_HIP((run_gemm<S, true, false, false>(s.dtype, Tn, f, h, dY, h, B, f, epi_b1, st)));
  }
  TPMLP_TRY(record(ev, 1, st));
  // B5: db1 = sum of the column partials
  if (f > 0) {
    hipLaunchKernelGGL((db1_finish_kernel<S, ACC>), dim3((unsigned)ceil_div(f, 32)), dim3(256), 0, st, part,
                       w.part_tiles, f, db1);
    TPMLP_HIP(hipGetLastError());
  }
  TPMLP_TRY(record(ev, 2, st));
  // B2 + B3 paired: with f = h, dB = H^T dY and dA = X^T dZ have one shape
  // and pitches; where each alone would be a launch of at most half a wave
  // (split into k-ranges), they run as one launch, unsplit (pair_fits).
  // Their events then bracket both in B2's interval; B3's is empty.
  const bool paired = !bt && H && f == h && !(room && (w.stage_b2 || w.stage_b3)) &&
                      pair_fits(s.dtype, f, h, Tn, false);
  if (paired) {
    TPMLP_TRY(record(ev, 3, st));
    TPMLP_TRY(record(ev, 4, st));
    TPMLP_HIP((run_gemm_pair<S, false, false>(f, h, Tn, H, dY, epi_dB(), X, dZ, epi_dA(), f, h, st)));
    TPMLP_TRY(record(ev, 5, st));
    TPMLP_TRY(record(ev, 6, st));
    TPMLP_TRY(record(ev, 7, st));
  } else {
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
  }
  TPMLP_TRY(record(ev, 8, st));
  // B4: dXp = dZ A_i^T; Q[k=f][n=h] = A_i[n][k] is k-contiguous
  TPMLP_HIP((run_gemm<S, true, true, false>(s.dtype, Tn, h, f, dZ, f, A, f, EpiStore<S>{(T*)dXp, h}, st, tail, tcap)));
  TPMLP_TRY(record(ev, 9, st));
  return TPMLP_OK;
}

template <class S, bool PK, bool QK>
hipError_t planned_gemm_t(int dtype, int64_t M, int64_t N, int64_t K, const void* p, int64_t ldp,
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
hipError_t planned_gemm_s(int dtype, bool pk, bool qk, int64_t M, int64_t N, int64_t K, const void* p,
                                 int64_t ldp, const void* q, int64_t ldq, void* out, int64_t ldo, const void* bias,
                                 float* tail_ws, size_t tail_cap, hipStream_t st) {
  if (pk && qk) return planned_gemm_t<S, true, true>(dtype, M, N, K, p, ldp, q, ldq, out, ldo, bias, tail_ws, tail_cap, st);
  if (pk) return planned_gemm_t<S, true, false>(dtype, M, N, K, p, ldp, q, ldq, out, ldo, bias, tail_ws, tail_cap, st);
  if (qk) return planned_gemm_t<S, false, true>(dtype, M, N, K, p, ldp, q, ldq, out, ldo, bias, tail_ws, tail_cap, st);
  return planned_gemm_t<S, false, false>(dtype, M, N, K, p, ldp, q, ldq, out, ldo, bias, tail_ws, tail_cap, st);
}

}  // namespace tpmlp

// Explicit instantiations of the launch sequences for storage type S:
// TPMLP_MLP_INSTANCES(, S) defines them, TPMLP_MLP_INSTANCES(extern, S)
// declares them in the translation units that only call them.
#define TPMLP_MLP_INSTANCES(PREFIX, S)                                                                              \
  namespace tpmlp {                                                                                                 \
  PREFIX template int fwd_impl<S>(const tpmlp_shape&, const void*, const void*, const void*, const void*, void*,   \
                                  void*, void*, void*, size_t, hipStream_t, void* const*, const RowSlices*);       \
  PREFIX template int bwd_impl<S, false>(const tpmlp_shape&, const void*, const void*, const void*, const void*,    \
                                         const void*, const void*, void*, void*, void*, void*, void*, const BwdWs&, \
                                         void*, size_t, hipStream_t, void* const*);                                \
  PREFIX template int bwd_impl<S, true>(const tpmlp_shape&, const void*, const void*, const void*, const void*,     \
                                        const void*, const void*, void*, void*, void*, void*, void*, const BwdWs&,  \
                                        void*, size_t, hipStream_t, void* const*);                                 \
  PREFIX template int recompute_z<S>(const tpmlp_shape&, const void*, const void*, const void*, void*, const RcWs&, \
                                     char*, hipStream_t, void* const*);                                            \
  }
#define TPMLP_GEMM_INSTANCES(PREFIX, S)                                                                              \
  namespace tpmlp {                                                                                                 \
  PREFIX template hipError_t planned_gemm_s<S>(int, bool, bool, int64_t, int64_t, int64_t, const void*, int64_t,    \
                                              const void*, int64_t, void*, int64_t, const void*, float*, size_t,    \
                                              hipStream_t);                                                        \
  }
