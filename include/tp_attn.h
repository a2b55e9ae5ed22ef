/*
 * tp_attn.h - one tensor-parallel rank's share of a Transformer
 * self-attention block, forward and backward, on an AMD Instinct MI355X
 * (gfx950). Built into the same library as tp_mlp.h and sharing its status
 * codes and dtype codes (tpmlp_status, tpmlp_dtype).
 *
 * The operation. Tensor parallelism splits the Q, K and V projections by
 * output columns and the output projection by input rows ("Megatron-LM
 * overview", section 2.2, the attention layer's QKV computation split over
 * devices; "Understanding the Megatron-LM architecture: how 3D parallelism
 * assigns roles", section 1, W_Q, W_K, W_V column-split and the attention
 * output projection row-split). Rank i owns n_i = heads of the layer's heads,
 * each of width d = head_dim, q = n_i d:
 *   Wqkv [hidden, 3q]   its heads' Q, K and V columns, laid out
 *                       [Q heads | K heads | V heads], head j's d columns
 *                       contiguous inside each block
 *   bqkv [3q]           their bias
 *   Wo   [q, hidden]    the rows of the output projection that read its heads
 * With T = batch * seq tokens (row b * seq + t is position t of sequence b):
 *   QKV = X Wqkv + bqkv                               [T, 3q]  kept for backward
 *   per sequence b and head j, with Q_bj, K_bj, V_bj the [seq, d] blocks:
 *     S  = Q_bj K_bj^T / sqrt(d), keys after the query masked out when
 *          causal ("Training GPT-2 with Megatron-LM", section 6.2, the
 *          fused_softmax switch: scale, mask and softmax as one step)
 *     P_bj = softmax(S) along the keys                [seq, seq] kept for backward
 *     O_bj = P_bj V_bj  -> columns j d .. j d + d - 1 of O   [T, q] kept
 *   Yp  = O Wo                                        [T, hidden] partial: sum
 *                                                     over ranks, + the output
 *                                                     bias, are the caller's
 * Backward, given dY [T, hidden] (the same on every rank):
 *   dO = dY Wo^T, dWo = O^T dY, dV = P^T dO, dP = dO V^T,
 *   dS = P * (dP - rowsum(P * dP)) / sqrt(d), dQ = dS K, dK = dS^T Q,
 *   dQKV = [dQ | dK | dV], dWqkv = X^T dQKV, dbqkv = column sums of dQKV,
 *   dXp = dQKV Wqkv^T (partial over ranks).
 * No dropout is applied.
 *
 * Conventions (as in tp_mlp.h): dense row-major tensors in the storage
 * dtype (fp16 or bf16 only; fp32 is TPMLP_ERR_DTYPE), fp32 accumulation,
 * every 16-bit result rounded once to nearest-even (the probabilities P and
 * the score gradients dS are rounded to storage before they enter the next
 * products); DEVICE pointers, 16-byte aligned; caller-owned buffers and
 * stream; asynchronous; outputs fully overwritten and not overlapping any
 * input or each other (TPMLP_ERR_ALIAS); validation errors return before
 * anything is enqueued; bitwise deterministic (no atomics). batch, seq,
 * hidden, heads and head_dim must be positive, and seq, hidden and head_dim
 * multiples of 8 (TPMLP_ERR_ALIGN); batch * heads * seq * seq must stay
 * below 2^40 (TPMLP_ERR_SHAPE).
 */
#ifndef TP_ATTN_H
#define TP_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include "tp_mlp.h"

#ifdef __cplusplus
extern "C" {
#endif

/* One rank's attention share. heads: this rank's heads (n_i). */
typedef struct {
  int64_t batch;
  int64_t seq;
  int64_t hidden;
  int64_t heads;
  int64_t head_dim;
  int32_t dtype;  /* TPMLP_F16 or TPMLP_BF16 */
  int32_t causal; /* nonzero: keys after the query are masked out */
} tpattn_shape;

/*
 * Workspace bytes (16-byte aligned device memory the caller owns; contents
 * on entry ignored; must not overlap any tensor argument):
 *   forward:  fp32 scores [batch*heads][seq][seq];
 *   backward: fp32 row terms rowsum(dO * O) [batch*heads][seq], dS
 *             [batch*heads][seq][seq] in the storage dtype, dO [T, q], fp32
 *             per-256-row column partials of dQKV for dbqkv, and fp32
 *             k-split partial sums of the projections' GEMMs.
 *   The forward's score buffer also holds the output projection's k-split
 *   partials, once the scores are consumed.
 * 0 on an invalid shape.
 */
size_t tp_attn_fwd_workspace_bytes(const tpattn_shape* shape);
size_t tp_attn_bwd_workspace_bytes(const tpattn_shape* shape);

/*
 * Forward of one rank.
 *   X    [T, hidden]                 in
 *   Wqkv [hidden, 3q], bqkv [3q]     in
 *   Wo   [q, hidden]                 in
 *   QKV  [T, 3q]                     out (kept for the backward)
 *   P    [batch*heads, seq, seq]     out, softmax probabilities of sequence b,
 *                                    head j at index b*heads + j (kept)
 *   O    [T, q]                      out (kept)
 *   Yp   [T, hidden]                 out, partial over ranks (no output bias)
 *   ws, ws_bytes                     at least tp_attn_fwd_workspace_bytes
 *                                    (TPMLP_ERR_WORKSPACE otherwise)
 */
int tp_attn_fwd(const tpattn_shape* shape,
                const void* X, const void* Wqkv, const void* bqkv, const void* Wo,
                void* QKV, void* P, void* O, void* Yp,
                void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of one rank.
 *   dY [T, hidden]                   in
 *   X, Wqkv, Wo                      in, as in tp_attn_fwd
 *   QKV, P, O                        in, the forward's outputs
 *   dQKV  [T, 3q]                    out
 *   dXp   [T, hidden]                out, partial over ranks
 *   dWqkv [hidden, 3q], dbqkv [3q]   out
 *   dWo   [q, hidden]                out
 *   ws, ws_bytes                     at least tp_attn_bwd_workspace_bytes
 */
int tp_attn_bwd(const tpattn_shape* shape,
                const void* dY, const void* X, const void* Wqkv, const void* Wo,
                const void* QKV, const void* P, const void* O,
                void* dQKV, void* dXp, void* dWqkv, void* dbqkv, void* dWo,
                void* ws, size_t ws_bytes, void* stream);

/*
 * Fused path: the same rank's share, with the attention core computed one
 * block of keys at a time on chip so that nothing of size seq x seq is
 * stored (the "flash" form of attention: an online softmax with a running
 * maximum and sum per query row). The forward keeps, per (sequence, head)
 * pair z = b * heads + j and query t, the log-sum-exp of the row's scaled,
 * masked scores,
 *   LSE[z][t] = log sum_{visible k} exp(S[t][k])   (fp32, natural log),
 * instead of P; the backward recomputes P[t][k] = exp(S[t][k] - LSE[z][t])
 * from it. Results equal those of tp_attn_fwd / tp_attn_bwd up to rounding
 * (the probabilities enter P V unnormalized, scaled by the row sum at the
 * end). Bitwise deterministic (no atomics).
 * Shapes: as above, without the sequence cap and without the
 * batch * heads * seq * seq bound; head_dim <= 128 (TPMLP_ERR_SHAPE).
 *
 * Workspace bytes (0 on an invalid shape):
 *   forward:  a transposed copy of Wo (when the output projection runs on
 *             the large-tile engine, which then reads both operands
 *             k-contiguous), a transposed copy of Wqkv (when the QKV
 *             projection runs on that engine's 256 x 256 tiles, whose
 *             16x16 MFMA form reads k-contiguous operands only) and the
 *             output projection's k-split partials, 256 at least;
 *   backward: fp32 row terms rowsum(dO * O) [batch*heads][seq], dO [T, q],
 *             fp32 per-256-row column partials of dQKV for dbqkv, and fp32
 *             k-split partials of the projections' GEMMs.
 */
size_t tp_attn_flash_fwd_workspace_bytes(const tpattn_shape* shape);
size_t tp_attn_flash_bwd_workspace_bytes(const tpattn_shape* shape);

/*
 * Fused forward of one rank: as tp_attn_fwd, with
 *   LSE  [batch*heads, seq] fp32     out (kept for the backward) in place of P.
 */
int tp_attn_flash_fwd(const tpattn_shape* shape,
                      const void* X, const void* Wqkv, const void* bqkv, const void* Wo,
                      void* QKV, void* LSE, void* O, void* Yp,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * Fused backward of one rank: as tp_attn_bwd, reading the forward's LSE
 * (fp32 [batch*heads, seq]) in place of P.
 */
int tp_attn_flash_bwd(const tpattn_shape* shape,
                      const void* dY, const void* X, const void* Wqkv, const void* Wo,
                      const void* QKV, const void* LSE, const void* O,
                      void* dQKV, void* dXp, void* dWqkv, void* dbqkv, void* dWo,
                      void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TP_ATTN_H */
