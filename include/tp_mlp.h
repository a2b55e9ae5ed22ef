/*
 * tp_mlp.h - one tensor-parallel rank's share of a Transformer MLP block,
 * forward and backward, on an AMD Instinct MI355X (gfx950).
 *
 * The operation. The MLP block is Y = GeLU(X A + b1) B (+ b2). Tensor
 * parallelism over P ranks splits the first linear by output columns and the
 * second by input rows ("Understanding the Megatron-LM architecture: how 3D
 * parallelism assigns roles", section 1, the column-split and row-split
 * bullets; "Megatron-LM overview", section 2.2). Rank i holds
 *   A_i  = A[:, i f : (i+1) f]   [hidden, f]
 *   b1_i = b1[i f : (i+1) f]     [f]
 *   B_i  = B[i f : (i+1) f, :]   [f, hidden]        with f = ffn / P,
 * computes its columns of the first linear on its own, and produces a
 * partial sum of the second linear that the caller reduces over ranks. The
 * bias add and the GeLU are one fused step ("Training GPT-2 with
 * Megatron-LM", section 6.2, fused_bias_gelu). GeLU is the tanh form
 *   gelu(x) = x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).
 *
 * Forward (tp_mlp_fwd), with T = tokens:
 *   Z_i  = X A_i + 1 b1_i^T        [T, f]   pre-activation, kept for backward
 *   H_i  = gelu(Z_i)               [T, f]   optional output
 *   Yp_i = H_i B_i                 [T, hidden] partial; sum over ranks (+ b2)
 * Backward (tp_mlp_bwd), given dY [T, hidden] (identical on every rank):
 *   dZ_i  = (dY B_i^T) * gelu'(Z_i)           [T, f]
 *   db1_i = sum over tokens of dZ_i           [f]
 *   dB_i  = H_i^T dY                          [f, hidden]
 *   dA_i  = X^T dZ_i                          [hidden, f]
 *   dXp_i = dZ_i A_i^T                        [T, hidden] partial; sum over ranks
 * The cross-rank sums (of Yp and dXp) and the second bias b2 are the
 * caller's; nothing here talks to another GPU.
 *
 * Conventions for every entry point below.
 *   - Tensors are dense, row-major, in the shapes above, all in the storage
 *     dtype of the shape (fp32, fp16 or bf16), inputs and outputs alike.
 *     Products accumulate in fp32; every 16-bit result is rounded once to
 *     nearest-even from its fp32 value.
 *   - Tensor pointers are DEVICE pointers on the current HIP device, 16-byte
 *     aligned. `stream` is a hipStream_t (NULL = the null stream). The
 *     caller owns every buffer and the stream; the library allocates nothing
 *     and keeps no per-call state, so calls from several threads are safe.
 *   - Calls are asynchronous: TPMLP_OK means the work was enqueued on
 *     `stream`. Outputs are fully overwritten (never accumulated into).
 *   - Dimensions may be 0. A product over an empty dimension is 0 (e.g.
 *     tokens == 0 gives dA = 0, dB = 0, db1 = 0); tensors with no elements
 *     are not touched. Nonzero dimensions must be multiples of 8 for fp16 /
 *     bf16 and of 4 for fp32, so that every row is 16-byte aligned.
 *   - Validation failures return before anything is enqueued and leave every
 *     output untouched. Outputs must not overlap each other or any input
 *     (TPMLP_ERR_ALIAS). A failed kernel launch returns TPMLP_ERR_HIP; HIP's
 *     sticky error state of the calling thread is read with hipGetLastError,
 *     so an error left pending by earlier, unrelated work may surface here.
 *   - Results are bitwise deterministic for a given shape, dtype and device:
 *     no floating-point atomics are used and every cross-workgroup sum runs
 *     in a fixed order.
 */
#ifndef TP_MLP_H
#define TP_MLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TPMLP_ABI_VERSION 8

typedef enum {
  TPMLP_F32 = 0,
  TPMLP_F16 = 1,
  TPMLP_BF16 = 2
} tpmlp_dtype;

typedef enum {
  TPMLP_OK = 0,
  TPMLP_ERR_NULL = 1,      /* a required pointer is NULL */
  TPMLP_ERR_SHAPE = 2,     /* negative dimension, or a size beyond the supported range */
  TPMLP_ERR_ALIGN = 3,     /* pointer not 16-byte aligned, or dimension not a multiple of 8 (4 for fp32) */
  TPMLP_ERR_DTYPE = 4,     /* dtype not one of tpmlp_dtype */
  TPMLP_ERR_WORKSPACE = 5, /* workspace smaller than tp_mlp_workspace_bytes() */
  TPMLP_ERR_HIP = 6,       /* a HIP call or kernel launch failed */
  TPMLP_ERR_ALIAS = 7,     /* an output overlaps an input or another output */
  TPMLP_ERR_SCRATCH = 8    /* tp_mlp_bwd_static: the shape needs more scratch than
                              TPMLP_STATIC_SCRATCH_BYTES */
} tpmlp_status;

/*
 * Shape of one rank's share: X [tokens, hidden], A_i [hidden, ffn_shard].
 *
 * layout: 0, or an OR of TPMLP_LAYOUT_B_T and TPMLP_LAYOUT_WEIGHTS_STAGED.
 * With TPMLP_LAYOUT_B_T the second weight is
 * passed as B_i^T [hidden, ffn_shard] (row-major), i.e. in the [out, in]
 * order of a linear layer's weight, and its gradient dB (or dB_main) is
 * written in that same [hidden, ffn_shard] order; every other tensor is as
 * described above. The pages fix only which dimension of the second weight
 * is split (its input rows), not the order in which a rank stores its block.
 *
 * TPMLP_LAYOUT_WEIGHTS_STAGED (read by tp_mlp_fwd and tp_mlp_fwd_sp; every
 * other call ignores it): the caller vouches that the forward workspace
 * `ws` already holds the k-contiguous copies of the weights that an earlier
 * tp_mlp_fwd or tp_mlp_fwd_sp call wrote there, with the same shape and
 * B_T bit, the same A_i and B_i contents, and the same ws pointer with
 * ws_bytes at least tp_mlp_fwd_workspace_bytes. The call then skips those
 * copies (the TA and TB transposes; their events are recorded back to
 * back) and reads the ones in the workspace. This serves gradient
 * accumulation over micro-batches ("Training GPT-2 with Megatron-LM",
 * section 4.3): the weights change only at the optimizer step, so the
 * first micro-batch's copies serve the rest. The library cannot check the
 * promise: with stale copies the results are those of the weights that
 * were copied. The rest of the workspace (k-split partial sums) is
 * rewritten by every call as before.
 *
 * Any other bit set is TPMLP_ERR_SHAPE. A zero-initialised struct (e.g.
 * {tokens, hidden, ffn_shard, dtype}) is the default layout.
 */
#define TPMLP_LAYOUT_B_T 1
#define TPMLP_LAYOUT_WEIGHTS_STAGED 2
typedef struct {
  int64_t tokens;
  int64_t hidden;
  int64_t ffn_shard;
  int32_t dtype;  /* tpmlp_dtype */
  int32_t layout; /* 0, or TPMLP_LAYOUT_B_T | TPMLP_LAYOUT_WEIGHTS_STAGED */
} tpmlp_shape;

/* TPMLP_ABI_VERSION of the built library. */
int tp_mlp_abi_version(void);

/* Static, human-readable name of a tpmlp_status value (never NULL). */
const char* tp_mlp_status_string(int status);

/*
 * Device workspace. The library allocates nothing; both passes take a
 * caller-owned workspace (16-byte aligned, contents on entry ignored, not
 * overlapping any tensor argument).
 *
 * tp_mlp_fwd_workspace_bytes: bytes with which tp_mlp_fwd stages
 * k-contiguous copies of A_i and B_i for the GEMMs that read them faster
 * that way, plus room for fp32 partial sums of a k-split last wave of
 * output tiles (below) (0 if this shape needs neither). tp_mlp_fwd
 * accepts any size: with less than this (or NULL) it reads the weights in
 * place and splits nothing, slower.
 *
 * k-split last wave: when a GEMM's output tiles leave a last wave that
 * would occupy at most half the compute units, each of those tiles is
 * computed as up to four k-ranges whose fp32 sums are added in a fixed
 * order (results stay deterministic, but differ in the last bits from an
 * unsplit run). Only plain-store GEMMs (the second forward GEMM, dB, dA,
 * dXp) split, and only with the full workspace; dB and dA do not where
 * tp_mlp_bwd runs them as one launch (see there).
 *
 * tp_mlp_workspace_bytes: bytes for tp_mlp_bwd. Flags:
 *   TPMLP_WS_DZ       room for dZ_i as well, for callers that pass dZ = NULL;
 *   TPMLP_WS_MINIMAL  only what tp_mlp_bwd requires (fp32 per-tile column
 *                     partials of dZ for db1, and dZ if TPMLP_WS_DZ);
 *   TPMLP_WS_RECOMPUTE the size for tp_mlp_bwd_recompute: room for the
 *                     recomputed Z_i (and a staged A_i^T) in front of
 *                     what the other flags ask for.
 * Without TPMLP_WS_MINIMAL the size also holds k-contiguous copies of H_i,
 * dY, X and dZ_i (each [rows][tokens]) for the weight-gradient GEMMs (and,
 * with TPMLP_LAYOUT_B_T, of B_i [ffn_shard][hidden] for the dZ GEMM) and
 * the k-split partial sums; tp_mlp_bwd uses them when ws_bytes reaches that
 * size, and otherwise reads the operands in place and splits nothing
 * (slower). A workspace below the minimal size is TPMLP_ERR_WORKSPACE.
 * Both return 0 and set nothing on an invalid shape.
 */
#define TPMLP_WS_DZ 1u
#define TPMLP_WS_MINIMAL 2u
#define TPMLP_WS_RECOMPUTE 4u
size_t tp_mlp_fwd_workspace_bytes(const tpmlp_shape* shape);
size_t tp_mlp_workspace_bytes(const tpmlp_shape* shape, unsigned flags);

/*
 * Forward of one rank (Z_i, optional H_i, partial Yp_i); see the top of this
 * file for the operation and conventions.
 *   X  [tokens, hidden]    in
 *   A  [hidden, ffn_shard] in   (A_i)
 *   b1 [ffn_shard]         in   (b1_i)
 *   B  [ffn_shard, hidden] in   (B_i; [hidden, ffn_shard] = B_i^T with
 *                               TPMLP_LAYOUT_B_T)
 *   Z  [tokens, ffn_shard] out  pre-activation X A_i + b1_i (bias included)
 *   H  [tokens, ffn_shard] out, may be NULL: gelu(Z_i). When NULL, the second
 *                          GEMM applies the GeLU to Z_i while loading it.
 *   Yp [tokens, hidden]    out  H_i B_i (partial over ranks, no b2)
 *   ws, ws_bytes           workspace (see tp_mlp_fwd_workspace_bytes); may
 *                          be NULL / 0.
 *   events: NULL, or 5 hipEvent_t recorded on `stream`: before the first
 *           kernel and after each of: A_i transpose (TA), first GEMM (F1),
 *           B_i transpose (TB), second GEMM (F2). A transpose that does not
 *           run leaves its two events back to back (TB never runs with
 *           TPMLP_LAYOUT_B_T: B_i^T is already k-contiguous for F2).
 *           A NULL entry is skipped (each record between two kernels
 *           costs the stream a few microseconds of idle time). The same
 *           holds for the events of every entry point below.
 */
int tp_mlp_fwd(const tpmlp_shape* shape,
               const void* X, const void* A, const void* b1, const void* B,
               void* Z, void* H, void* Yp,
               void* ws, size_t ws_bytes,
               void* stream, void* const* events);

/*
 * Forward of one rank under sequence parallelism: the tokens of X are split
 * over the ranks as well ("Training GPT-2 with Megatron-LM", section 5.1,
 * the --sequence-parallel switch), so rank r holds only token rows
 * [r T/n, (r+1) T/n) of X. The column-split first linear needs every token,
 * which the pages obtain by all-gathering the input ("Understanding the
 * Megatron-LM architecture: how 3D parallelism assigns roles", section 1,
 * the row-split item: "All-Gather the input, or All-Reduce the result").
 * Here the gather is folded into the first GEMM's operand loads: it reads
 * each token row straight from the slice that holds it, and no gathered copy
 * of X is made. Everything else is tp_mlp_fwd; the outputs Z, H and Yp cover
 * all T tokens, and rank r's reduce-scatter of Yp over the ranks is
 * tp_mlp_reduce_partials over rows [r T/n, (r+1) T/n).
 *   nslices     1 .. 16 (TPMLP_ERR_SHAPE otherwise); tokens must be a
 *               multiple of nslices (TPMLP_ERR_SHAPE)
 *   X_slices    HOST array of nslices DEVICE pointers, slice i holding token
 *               rows [i T/n, (i+1) T/n) of X, each [tokens / nslices, hidden],
 *               16-byte aligned; outputs may not overlap any slice
 *   others      as in tp_mlp_fwd (same workspace size, same 5 events)
 * fp16 and bf16 only (TPMLP_ERR_DTYPE for fp32). The results are bitwise
 * those of tp_mlp_fwd on the gathered X.
 */
int tp_mlp_fwd_sp(const tpmlp_shape* shape, int nslices, const void* const* X_slices,
                  const void* A, const void* b1, const void* B,
                  void* Z, void* H, void* Yp,
                  void* ws, size_t ws_bytes,
                  void* stream, void* const* events);

/*
 * Backward of one rank; see the top of this file for the operation.
 *   dY  [tokens, hidden]    in   output gradient (same on every rank)
 *   X, A, B                 in   as in tp_mlp_fwd
 *   Z   [tokens, ffn_shard] in   the forward's Z_i
 *   H   [tokens, ffn_shard] in, may be NULL: the forward's H_i. When NULL,
 *                           gelu(Z_i) is recomputed from Z_i.
 *   dZ  [tokens, ffn_shard] out, may be NULL: dZ_i. When NULL it is kept in
 *                           the workspace (size it with TPMLP_WS_DZ).
 *   dXp [tokens, hidden]    out  dZ_i A_i^T (partial over ranks)
 *   dA  [hidden, ffn_shard] out  X^T dZ_i
 *   dB  [ffn_shard, hidden] out  H_i^T dY ([hidden, ffn_shard] = dY^T H_i
 *                                with TPMLP_LAYOUT_B_T)
 *   db1 [ffn_shard]         out  column sums of dZ_i
 *   ws, ws_bytes            workspace of at least
 *                           tp_mlp_workspace_bytes(shape, TPMLP_WS_MINIMAL |
 *                           (dZ == NULL ? TPMLP_WS_DZ : 0)) bytes; may be
 *                           NULL when that is 0.
 *   events: NULL, or 10 hipEvent_t recorded on `stream`: before the first
 *           kernel and after each of: dZ GEMM with the db1 column partials
 *           (B1), db1 finish (B5), H_i transpose (TH), dY transpose (TdY),
 *           dB GEMM (B2), X transpose (TX), dZ_i transpose (TdZ), dA GEMM
 *           (B3), dXp GEMM (B4). A transpose that does not run leaves its
 *           two events back to back. With TPMLP_LAYOUT_B_T and the staged
 *           workspace, B1's interval also holds a transpose of B_i^T into
 *           the workspace, from which the dZ GEMM reads B_i k-contiguous.
 *           Where dB and dA run as one launch (below), B2's interval holds
 *           both and B3's two events are back to back.
 * dB and dA as one launch: with ffn_shard == hidden, H_i kept, the default
 * layout and operands read in place, the two weight-gradient GEMMs have one
 * shape; where each alone would fill at most half of the compute units,
 * they run as one launch of both GEMMs' output tiles, each over the whole
 * token reduction (no k-split partials for them).
 */
int tp_mlp_bwd(const tpmlp_shape* shape,
               const void* dY, const void* X, const void* A, const void* B,
               const void* Z, const void* H,
               void* dZ, void* dXp, void* dA, void* dB, void* db1,
               void* ws, size_t ws_bytes,
               void* stream, void* const* events);

/*
 * Backward that allocates nothing and takes no workspace: for callers that
 * cannot call hipMalloc or hand the library memory of its own (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Same operation, arguments, layout, events and error codes as
 * tp_mlp_bwd with a minimal workspace (TPMLP_WS_MINIMAL), minus ws and
 * ws_bytes; the results are bitwise those of that call.
 *   dZ  [tokens, ffn_shard] out, REQUIRED here (TPMLP_ERR_NULL if NULL):
 *                           there is no workspace to keep it in.
 * Its only scratch, the fp32 per-tile column partials of dZ_i that the db1
 * finish adds up, lives in a device array of TPMLP_STATIC_SCRATCH_BYTES
 * that the library defines once per GPU it runs on (held until the process
 * ends; its address is looked up once per device, on the first call made
 * with that device current). A shape whose partials need more returns
 * TPMLP_ERR_SCRATCH before anything is enqueued; the size they need is
 * tp_mlp_workspace_bytes(shape, TPMLP_WS_MINIMAL). Every call on one GPU
 * uses that GPU's one array: calls that overlap on the same GPU (several
 * streams or threads at once) race and give wrong results; serialise them.
 * Nothing in the array needs clearing: each call overwrites every partial
 * it reads.
 */
#define TPMLP_STATIC_SCRATCH_BYTES (32u << 20)
int tp_mlp_bwd_static(const tpmlp_shape* shape,
                      const void* dY, const void* X, const void* A, const void* B,
                      const void* Z, const void* H,
                      void* dZ, void* dXp, void* dA, void* dB, void* db1,
                      void* stream, void* const* events);

/*
 * Backward with selective recomputation: the forward's Z_i and H_i are not
 * kept; Z_i = X A_i + b1_i is recomputed here first (the forward's first
 * step, "Megatron-LM overview", section 3.3, activation checkpointing),
 * into the front of the workspace, and H_i is taken as gelu(Z_i) where it
 * is needed. Arguments as in tp_mlp_bwd, plus b1 [ffn_shard] in, minus Z
 * and H. ws: at least tp_mlp_workspace_bytes(shape, TPMLP_WS_RECOMPUTE |
 * TPMLP_WS_MINIMAL | (dZ == NULL ? TPMLP_WS_DZ : 0)) bytes (never NULL for
 * a nonempty shape); with TPMLP_WS_RECOMPUTE alone the transposed copies
 * are staged as in tp_mlp_bwd.
 *   events: NULL, or 12 hipEvent_t recorded on `stream`: before the first
 *           kernel, after the A_i transpose (TA), after the recomputing
 *           GEMM (F1), then as tp_mlp_bwd's events 1-9.
 * Results are bitwise those of tp_mlp_fwd (H not kept) followed by
 * tp_mlp_bwd with H = NULL.
 */
int tp_mlp_bwd_recompute(const tpmlp_shape* shape,
                         const void* dY, const void* X, const void* A, const void* b1, const void* B,
                         void* dZ, void* dXp, void* dA, void* dB, void* db1,
                         void* ws, size_t ws_bytes,
                         void* stream, void* const* events);

/*
 * Backward with gradient accumulation into fp32 main gradients: as
 * tp_mlp_bwd, except that the weight gradients of this micro-batch are
 * ADDED (beta = 1) to fp32 buffers the caller keeps across micro-batches,
 * without a rounding to the storage dtype on the way:
 *   dA_main  [hidden, ffn_shard] fp32   += X^T dZ_i
 *   dB_main  [ffn_shard, hidden] fp32   += H_i^T dY   ([hidden, ffn_shard]
 *                                              with TPMLP_LAYOUT_B_T)
 *   db1_main [ffn_shard]         fp32   += sum over tokens of dZ_i
 * (the pages train with fp16 products and fp32 master weights, "Megatron-LM
 * overview", section 3.1, and accumulate gradients over micro-batches,
 * "Training GPT-2 with Megatron-LM", section 4.3). dZ, dXp, the workspace
 * (sized with tp_mlp_workspace_bytes) and the 10 events are exactly as in
 * tp_mlp_bwd. The main gradients are read and written, never just written;
 * like the other outputs they must not overlap any input or each other.
 * For fp32 storage the products are the same fp32 FMAs as in tp_mlp_bwd.
 */
int tp_mlp_bwd_main_grad(const tpmlp_shape* shape,
                         const void* dY, const void* X, const void* A, const void* B,
                         const void* Z, const void* H,
                         void* dZ, void* dXp, float* dA_main, float* dB_main, float* db1_main,
                         void* ws, size_t ws_bytes,
                         void* stream, void* const* events);

/*
 * Gradient of the second bias b2, which the caller adds once after the sum
 * over ranks (so its gradient is the same on every rank, from the replicated
 * dY): db2[c] = sum over tokens t of dY[t][c]. The pages accumulate weight
 * gradients over micro-batches in fp32 master copies ("Training GPT-2 with
 * Megatron-LM", section 4.3; "Megatron-LM overview", section 3.1), hence
 * the accumulate form.
 *   dY   [tokens, hidden]   in
 *   db2  [hidden]           out: with accumulate == 0, in the storage dtype,
 *                           rounded once from the fp32 sum; with accumulate
 *                           != 0, an fp32 main gradient, db2 += the fp32 sum
 *   ws, ws_bytes            at least tp_mlp_db2_workspace_bytes (fp32
 *                           partial sums per 256 tokens; 0 for fp32 storage);
 *                           may be NULL when that is 0
 * The sum runs in a fixed order (256-token blocks, then blocks in order):
 * bitwise deterministic. tokens may be 0 (db2 = 0, or unchanged when
 * accumulating); more than 65535 x 256 tokens is TPMLP_ERR_SHAPE.
 * ffn_shard is not used but must be valid.
 */
size_t tp_mlp_db2_workspace_bytes(const tpmlp_shape* shape);
int tp_mlp_db2(const tpmlp_shape* shape, const void* dY, void* db2, int accumulate, void* ws, size_t ws_bytes,
               void* stream);

/*
 * Sum over ranks of the row-parallel partials, for P ranks whose partials
 * sit on this device: the arithmetic of the all-reduce that follows the
 * second linear ("Understanding the Megatron-LM architecture: how 3D
 * parallelism assigns roles", section 1, the row-split item), and, over one
 * rank's slice of rows, of the reduce-scatter that replaces it when the
 * sequence dimension is split as well ("Training GPT-2 with Megatron-LM",
 * section 5.1, the --sequence-parallel switch). For rows r in
 * [row_begin, row_end):
 *   out[r - row_begin][c] = round( sum_{i < nparts} parts[i][r][c] (+ bias[c]) )
 * with fp32 sums in the order i = 0, 1, ..., the bias added last and one
 * rounding to the storage dtype.
 *   shape       tokens (rows of each partial), hidden (columns) and dtype;
 *               ffn_shard is not used but must be valid
 *   nparts      1 .. 16 (TPMLP_ERR_SHAPE otherwise)
 *   parts       HOST array of nparts DEVICE pointers, each [tokens, hidden]
 *               (the forward's Yp or the backward's dXp of each rank)
 *   bias        [hidden] (b2 after the forward), or NULL for none
 *   row_begin, row_end   0 <= row_begin <= row_end <= tokens
 *               (TPMLP_ERR_SHAPE otherwise); all rows: 0, tokens
 *   out         [row_end - row_begin, hidden]; must not overlap any part or
 *               the bias (TPMLP_ERR_ALIAS: no in-place form)
 * Asynchronous on `stream` like the other calls; bitwise deterministic.
 */
#define TPMLP_MAX_PARTS 16
int tp_mlp_reduce_partials(const tpmlp_shape* shape, int nparts, const void* const* parts, const void* bias,
                           int64_t row_begin, int64_t row_end, void* out, void* stream);

/*
 * Tile-plan override, for tests and tuning only (production callers leave
 * it alone). It forces the GEMM engine of every 16-bit product and the CU
 * count the k-split planner assumes, so that small shapes exercise the
 * large-tile engines and their k-split paths. Process-wide; applies to
 * calls that start after it returns (workspace sizes included).
 *   tile      TPMLP_PLAN_AUTO (the planner's choice), TPMLP_PLAN_REG128 /
 *             TPMLP_PLAN_REG256 (register-staged 128x128 / 256x256 tiles),
 *             TPMLP_PLAN_DMA256 (direct-load 256x256), TPMLP_PLAN_DMA320
 *             (direct-load 256x320 where both operands are k-contiguous,
 *             256x256 elsewhere), TPMLP_PLAN_DMA320_M32 (as DMA320, with
 *             every direct-load tile on the 32x32x16 MFMA form; otherwise
 *             they run on the 16x16x32 form, except under the fp32
 *             main-gradient accumulation). A forced direct-load engine still yields
 *             to the register-staged 256x256 one where an operand exceeds
 *             its 32-bit offsets or GeLU is applied on load.
 *   tail_cus  CU count of the k-split plan, 1 .. 4096; 0 = the chip's 256.
 * Returns TPMLP_ERR_SHAPE for values out of range (nothing changes then).
 */
#define TPMLP_PLAN_AUTO 0
#define TPMLP_PLAN_REG128 1
#define TPMLP_PLAN_REG256 2
#define TPMLP_PLAN_DMA256 3
#define TPMLP_PLAN_DMA320 4
#define TPMLP_PLAN_DMA320_M32 5
int tp_mlp_debug_plan(int tile, int tail_cus);

#ifdef __cplusplus
}
#endif

#endif /* TP_MLP_H */
