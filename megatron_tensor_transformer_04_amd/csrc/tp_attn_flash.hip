// C ABI of the fused attention path (declared in include/tp_attn.h,
// tp_attn_flash_*): the same rank's share as tp_attn_fwd / tp_attn_bwd, with
// the per-head core (scores, softmax, P V and their backward) in the kernels
// of flash_attn.hpp, so that nothing of size seq x seq is stored. The
// forward keeps the per-row log-sum-exp L instead of P; the backward
// recomputes P from it. The projections and their gradients go through the
// MLP shard's GEMM planner (shard_gemm.hpp) as in the materialized path.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "tp_attn.h"
#include "attn_common.hpp"
#include "colsum.hpp"
#include "flash_attn.hpp"
#include "shard_gemm.hpp"

namespace tpmlp {
namespace {

using namespace attn;

// Forward workspace: [Wo^T [h][staged_transpose_ld(q)], when the output
// projection runs on the large-tile engine with both operands k-contiguous]
// [Wqkv^T [3q][staged_transpose_ld(h)], when the k-contiguous copy pays for
// the QKV projection (planned_gemm_stages_weight)] [the output
// projection's k-split partials]; 256 bytes at least, so that 0 keeps
// meaning an invalid shape.
struct FlashFwdWs {
  bool wot, wqkvt;
  size_t wqkvt_off, tail_off, total;
};

FlashFwdWs flash_fwd_layout(const AttnDims& a, int dtype) {
  FlashFwdWs w{};
  w.wot = planned_gemm_stages(dtype, a.T, a.h, a.q);
  w.wqkvt = planned_gemm_stages_weight(dtype, a.T, 3 * a.q, a.h);
  w.wqkvt_off = w.wot ? a256((size_t)(a.h * staged_transpose_ld(a.q)) * 2) : 0;
  w.tail_off = w.wqkvt_off + (w.wqkvt ? a256((size_t)(3 * a.q * staged_transpose_ld(a.h)) * 2) : 0);
  w.total = std::max<size_t>(256, w.tail_off + a256(planned_gemm_tail_bytes(dtype, a.T, a.h, a.q, w.wot)));
  return w;
}

size_t flash_fwd_ws(const AttnDims& a, int dtype) { return flash_fwd_layout(a, dtype).total; }

// Backward workspace: [D fp32 Z s][dO 16-bit T q][column partials of dQKV
// fp32 [T/256][3q]][k-split partials of the projections' plain-store GEMMs].
struct FlashBwdWs {
  size_t drow_off, do_off, part_off, tail_off, tail_bytes, total;
  int part_blk;
};

FlashBwdWs flash_bwd_layout(const AttnDims& a, int dtype) {
  FlashBwdWs w{};
  const int64_t T3 = 3 * a.q;
  w.drow_off = 0;
  w.do_off = a256((size_t)(a.Z * a.s) * 4);
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

flash::Args core_args(const AttnDims& a, int causal, const void* QKV) {
  flash::Args f{};
  f.qkv = static_cast<const uint16_t*>(QKV);
  f.s = a.s;
  f.ld3 = 3 * a.q;
  f.ldo = a.q;
  f.heads = (int)a.n;
  f.d = (int)a.d;
  f.q = (int)a.q;
  f.nblk = (int)cdiv(a.s, flash::kRows);
  f.Z = (int)a.Z;
  f.scale = a.scale;
  f.scale_log2 = flash::kLog2e * a.scale;
  f.causal = causal ? 1 : 0;
  f.one_bits = 0;
  return f;
}

template <class S>
int flash_fwd_impl(const AttnDims& a, int dtype, int causal, const void* X, const void* Wqkv, const void* bqkv,
                   const void* Wo, void* QKV, void* LSE, void* O, void* Yp, void* ws, size_t ws_bytes,
                   hipStream_t st) {
  const int64_t T3 = 3 * a.q;
  const FlashFwdWs w = flash_fwd_layout(a, dtype);
  char* wsb = static_cast<char*>(ws);
  // QKV = X Wqkv + bqkv: P = X [T,h] k-contiguous, Q = Wqkv [h,3q]
  // n-contiguous, or its copy Wqkv^T [3q][h] (k-contiguous) where that pays
  // (the 16x16 MFMA form reads k-contiguous operands only)
  if (w.wqkvt) {
    const int64_t ldt = staged_transpose_ld(a.h);
    ATTN_HIP(staged_transpose(Wqkv, wsb + w.wqkvt_off, a.h, T3, st));
    ATTN_HIP(planned_gemm(dtype, true, true, a.T, T3, a.h, X, a.h, wsb + w.wqkvt_off, ldt, QKV, T3, bqkv, nullptr,
                          0, st));
  } else {
    ATTN_HIP(planned_gemm(dtype, true, false, a.T, T3, a.h, X, a.h, Wqkv, T3, QKV, T3, bqkv, nullptr, 0, st));
  }
  flash::Args f = core_args(a, causal, QKV);
  f.lse = static_cast<float*>(LSE);
  f.out = static_cast<uint16_t*>(O);
  f.one_bits = dtype == TPMLP_BF16 ? 0x3F80u : 0x3C00u;  // 1.0
  ATTN_HIP(flash::launch_fwd<S>(f, st));
  // Yp = O Wo: P = O [T,q] k-contiguous; Q = Wo [q,h] is n-contiguous, so
  // where the large-tile engine runs it a transposed copy Wo^T [h][q] is
  // staged first (3 MB at the 2.4B shape), which lets it take the 320-wide
  // tiles (one wave of 256 x 320 there, against 1.25 of 256 x 256)
  if (w.wot) {
    const int64_t ldt = staged_transpose_ld(a.q);
    ATTN_HIP(staged_transpose(Wo, wsb, a.q, a.h, st));
    ATTN_HIP(planned_gemm(dtype, true, true, a.T, a.h, a.q, O, a.q, wsb, ldt, Yp, a.h, nullptr,
                          reinterpret_cast<float*>(wsb + w.tail_off), ws_bytes - w.tail_off, st));
  } else {
    ATTN_HIP(planned_gemm(dtype, true, false, a.T, a.h, a.q, O, a.q, Wo, a.h, Yp, a.h, nullptr,
                          reinterpret_cast<float*>(wsb + w.tail_off), ws_bytes - w.tail_off, st));
  }
  return TPMLP_OK;
}

template <class S>
int flash_bwd_impl(const AttnDims& a, int dtype, int causal, const void* dY, const void* X, const void* Wqkv,
                   const void* Wo, const void* QKV, const void* LSE, const void* O, void* dQKV, void* dXp,
                   void* dWqkv, void* dbqkv, void* dWo, void* ws, hipStream_t st) {
  using T = typename S::T;
  const int64_t T3 = 3 * a.q;
  const FlashBwdWs w = flash_bwd_layout(a, dtype);
  char* wsb = static_cast<char*>(ws);
  float* drow = reinterpret_cast<float*>(wsb + w.drow_off);
  T* dO = reinterpret_cast<T*>(wsb + w.do_off);
  float* part = reinterpret_cast<float*>(wsb + w.part_off);
  float* tail = reinterpret_cast<float*>(wsb + w.tail_off);
  // dO = dY Wo^T: Q[k=h][n=q] = Wo[n][k] k-contiguous
  ATTN_HIP(planned_gemm(dtype, true, true, a.T, a.q, a.h, dY, a.h, Wo, a.h, dO, a.q, nullptr, tail, w.tail_bytes, st));
  // dWo = O^T dY: P[m=q][k=T] = O[k][m], Q = dY [T,h]: both mn-contiguous
  ATTN_HIP(planned_gemm(dtype, false, false, a.q, a.h, a.T, O, a.q, dY, a.h, dWo, a.h, nullptr, tail, w.tail_bytes,
                        st));
  // D = rowsum(dO * O) per (pair, query)
  hipLaunchKernelGGL(softmax_rowdot_kernel<S>, dim3((unsigned)cdiv(a.T * a.n, 256)), dim3(256), 0, st, dO,
                     static_cast<const T*>(O), drow, a.T, a.s, (int)a.n, (int)a.d, a.q);
  ATTN_HIP(hipGetLastError());
  // dK, dV (K and V blocks of dQKV), then dQ (its Q block)
  flash::Args f = core_args(a, causal, QKV);
  f.dO = dO;
  f.D = drow;
  f.lse = const_cast<float*>(static_cast<const float*>(LSE));
  f.out = static_cast<uint16_t*>(dQKV);
  ATTN_HIP(flash::launch_bwd<S>(f, st));
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
using namespace tpmlp::attn;

extern "C" {

size_t tp_attn_flash_fwd_workspace_bytes(const tpattn_shape* shape) {
  if (check_attn_shape(shape, true) != TPMLP_OK) return 0;
  return flash_fwd_ws(dims(*shape), shape->dtype);
}

size_t tp_attn_flash_bwd_workspace_bytes(const tpattn_shape* shape) {
  if (check_attn_shape(shape, true) != TPMLP_OK) return 0;
  return flash_bwd_layout(dims(*shape), shape->dtype).total;
}

int tp_attn_flash_fwd(const tpattn_shape* shape, const void* X, const void* Wqkv, const void* bqkv, const void* Wo,
                      void* QKV, void* LSE, void* O, void* Yp, void* ws, size_t ws_bytes, void* stream) {
  const int rc = check_attn_shape(shape, true);
  if (rc != TPMLP_OK) return rc;
  const AttnDims a = dims(*shape);
  const size_t e = 2, need = tp_attn_flash_fwd_workspace_bytes(shape);
  const Span2 in[4] = {{X, (size_t)(a.T * a.h) * e}, {Wqkv, (size_t)(a.h * 3 * a.q) * e},
                       {bqkv, (size_t)(3 * a.q) * e}, {Wo, (size_t)(a.q * a.h) * e}};
  const Span2 out[5] = {{QKV, (size_t)(a.T * 3 * a.q) * e}, {LSE, (size_t)(a.Z * a.s) * 4},
                        {O, (size_t)(a.T * a.q) * e}, {Yp, (size_t)(a.T * a.h) * e}, {ws, std::min(need, ws_bytes)}};
  const int bc = check_spans(in, 4, out, 5);
  if (bc != TPMLP_OK) return bc;
  if (ws_bytes < need) return TPMLP_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (shape->dtype == TPMLP_F16)
    return flash_fwd_impl<StoreF16>(a, shape->dtype, shape->causal, X, Wqkv, bqkv, Wo, QKV, LSE, O, Yp, ws, need, st);
  return flash_fwd_impl<StoreBF16>(a, shape->dtype, shape->causal, X, Wqkv, bqkv, Wo, QKV, LSE, O, Yp, ws, need, st);
}

int tp_attn_flash_bwd(const tpattn_shape* shape, const void* dY, const void* X, const void* Wqkv, const void* Wo,
                      const void* QKV, const void* LSE, const void* O, void* dQKV, void* dXp, void* dWqkv,
                      void* dbqkv, void* dWo, void* ws, size_t ws_bytes, void* stream) {
  const int rc = check_attn_shape(shape, true);
  if (rc != TPMLP_OK) return rc;
  const AttnDims a = dims(*shape);
  const size_t e = 2, need = tp_attn_flash_bwd_workspace_bytes(shape);
  const size_t Th = (size_t)(a.T * a.h) * e, T3 = (size_t)(a.T * 3 * a.q) * e, h3 = (size_t)(a.h * 3 * a.q) * e,
               qh = (size_t)(a.q * a.h) * e;
  const Span2 in[7] = {{dY, Th}, {X, Th}, {Wqkv, h3}, {Wo, qh}, {QKV, T3}, {LSE, (size_t)(a.Z * a.s) * 4},
                       {O, (size_t)(a.T * a.q) * e}};
  const Span2 out[6] = {{dQKV, T3}, {dXp, Th}, {dWqkv, h3}, {dbqkv, (size_t)(3 * a.q) * e}, {dWo, qh},
                        {ws, std::min(need, ws_bytes)}};
  const int bc = check_spans(in, 7, out, 6);
  if (bc != TPMLP_OK) return bc;
  if (ws_bytes < need) return TPMLP_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (shape->dtype == TPMLP_F16)
    return flash_bwd_impl<StoreF16>(a, shape->dtype, shape->causal, dY, X, Wqkv, Wo, QKV, LSE, O, dQKV, dXp, dWqkv,
                                    dbqkv, dWo, ws, st);
  return flash_bwd_impl<StoreBF16>(a, shape->dtype, shape->causal, dY, X, Wqkv, Wo, QKV, LSE, O, dQKV, dXp, dWqkv,
                                   dbqkv, dWo, ws, st);
}

}  // extern "C"
