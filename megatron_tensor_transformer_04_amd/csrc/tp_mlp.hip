// C ABI of the tensor-parallel MLP shard (declared in include/tp_mlp.h):
// argument validation, workspace sizes and dispatch over the storage type to
// the launch sequences of mlp_impl.hpp (instantiated per type in
// mlp_f32.hip, mlp_f16.hip and mlp_bf16.hip); the static device scratch of
// the allocation-free backward; db2 (column sums of dY); and
// tp_mlp_reduce_partials, which sums the row-parallel partials of P ranks
// held on this device (plus b2), over all rows or one rank's slice of rows.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tp_mlp.h"
#include "colsum.hpp"
#include "mlp_impl.hpp"
#include "reduce.hpp"
#include "shard_gemm.hpp"

TPMLP_MLP_INSTANCES(extern, tpmlp::StoreF32)
TPMLP_MLP_INSTANCES(extern, tpmlp::StoreF16)
TPMLP_MLP_INSTANCES(extern, tpmlp::StoreBF16)
TPMLP_GEMM_INSTANCES(extern, tpmlp::StoreF16)
TPMLP_GEMM_INSTANCES(extern, tpmlp::StoreBF16)

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

}  // namespace

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

bool planned_gemm_stages(int dtype, int64_t M, int64_t N, int64_t K) { return stages(dtype, M, N, K); }

bool planned_gemm_stages_weight(int dtype, int64_t M, int64_t N, int64_t K) {
  return stages_weight(dtype, M, N, K);
}

hipError_t staged_transpose(const void* in, void* out, int64_t R, int64_t C, hipStream_t st) {
  // the transpose moves 16-bit values: the storage type only names them
  return run_transpose<StoreBF16, false>(in, out, R, C, st);
}

int64_t staged_transpose_ld(int64_t R) { return staged_ld(R); }

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

int tp_mlp_fwd_sp(const tpmlp_shape* shape, int nslices, const void* const* X_slices, const void* A,
                  const void* b1, const void* B, void* Z, void* H, void* Yp, void* ws, size_t ws_bytes, void* stream,
                  void* const* events) {
  TPMLP_TRY(check_shape(shape));
  const tpmlp_shape& s = *shape;
  if (s.dtype == TPMLP_F32) return TPMLP_ERR_DTYPE;
  if (nslices < 1 || nslices > kMaxSlices || s.tokens % nslices) return TPMLP_ERR_SHAPE;
  if (!X_slices) return TPMLP_ERR_NULL;
  const size_t e = elt_size(s.dtype);
  const int64_t rows = s.tokens / nslices;
  const size_t Th = (size_t)(s.tokens * s.hidden) * e, hf = (size_t)(s.hidden * s.ffn_shard) * e,
               Tf = (size_t)(s.tokens * s.ffn_shard) * e, fb = (size_t)s.ffn_shard * e, sb = (size_t)(rows * s.hidden) * e;
  Span in[kMaxSlices + 3];
  bool in_req[kMaxSlices + 3];
  for (int i = 0; i < nslices; ++i) {
    in[i] = Span{X_slices[i], sb};
    in_req[i] = true;
  }
  in[nslices] = Span{A, hf};
  in[nslices + 1] = Span{b1, fb};
  in[nslices + 2] = Span{B, hf};
  for (int i = 0; i < 3; ++i) in_req[nslices + i] = true;
  const Span out[4] = {{Z, Tf}, {H, Tf}, {Yp, Th}, {ws, ws ? ws_bytes : 0}};
  const bool out_req[4] = {true, false, true, false};
  TPMLP_TRY(check_buffers(in, nslices + 3, in_req, out, 4, out_req));
  RowSlices xs{};
  for (int i = 0; i < nslices; ++i) xs.p[i] = static_cast<const uint16_t*>(X_slices[i]);
  xs.rows = rows > 0 ? rows : 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s.dtype == TPMLP_F16) return fwd_impl<StoreF16>(s, nullptr, A, b1, B, Z, H, Yp, ws, ws_bytes, st, events, &xs);
  return fwd_impl<StoreBF16>(s, nullptr, A, b1, B, Z, H, Yp, ws, ws_bytes, st, events, &xs);
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
  if (tile < TPMLP_PLAN_AUTO || tile > TPMLP_PLAN_DMA320_M32 || tail_cus < 0 || tail_cus > 4096) return TPMLP_ERR_SHAPE;
  g_plan_tile.store(tile, std::memory_order_relaxed);
  g_plan_mf16.store(tile != TPMLP_PLAN_DMA320_M32, std::memory_order_relaxed);
  g_plan_cus.store(tail_cus, std::memory_order_relaxed);
  return TPMLP_OK;
}

}  // extern "C"
