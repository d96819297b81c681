/*
 * tp_mlp.h -- one tensor-parallel rank of the Megatron paired MLP block on
 * MI355X (gfx950).  C ABI of libtpmlp.so.
 *
 * The method (column-parallel up-projection, elementwise activation on the
 * local shard, row-parallel down-projection to a full-shape partial sum, one
 * reduction of the partials, output bias added once after it, and the matching
 * sharded backward) is described by:
 *   - "02 -- Tensor Parallelism" (project-fortress roadmap), sections
 *     "Column-parallel", "Row-parallel" and "The MLP pairing";
 *   - "Tensor Parallelism's Communication Boundary" (aryanputta.com), sections
 *     "Follow the coordinates" and the bias caveat under "Count the object,
 *     then the collective";
 *   - "Parallelism Strategies #1 - Tensor Parallelism" (deeplearningresearch
 *     substack), the sharded backward derivation;
 *   - "Tensor and sequence parallelism" (AI infra handbooks), the f / g
 *     operator table;
 *   - "Megatron-LM: Tensor Parallelism" (vanos001 placement prep), section
 *     "MLP Block".
 *
 * Conventions for every entry point
 *   Layout     All matrices are dense, row-major, math layout (input dim
 *              first): X [N, h], W1_i and Wg_i [h, F_i], W2_i [F_i, h], with
 *              N = n_tokens, h = hidden, F_i = ffn / t.  Row strides equal the
 *              row lengths (no padding).
 *   Types      Activations and weights are bfloat16 (passed as void*);
 *              weight gradients and db2 are float32.  Every product
 *              accumulates in float32; bf16 outputs are rounded to nearest
 *              even once.
 *   Pointers   Every pointer is a DEVICE pointer, 16-byte aligned, except
 *              the shape structs and the HOST arrays of device pointers that
 *              the local reductions take (tp_mlp_reduce_partials_local,
 *              tp_mlp_reduce_scatter_local, tp_mlp_all_gather_local,
 *              tp_sp_reduce_scatter_layernorm_local, tp_sp_sum_grads_local).
 *              h and F_i must be multiples of 8.
 *   Overlap    An output may not overlap another output, an input or the
 *              workspace in use, except where an entry point states that it
 *              may coincide exactly with one (in-place forms); such calls
 *              return TP_MLP_ERR_INVALID_ARG.
 *   Extents    Every bf16 operand of a GEMM (X, a weight shard, A_i, dU_i,
 *              the attention projections' operands) is at most 4 GiB - 256
 *              bytes: the kernels address each through a 32-bit buffer
 *              descriptor.  The streaming entry points (local reductions,
 *              reduce-scatter, all-gather, bias gradient) take cols <= 2^33
 *              and rows * cols <= 2^50.  Larger calls return
 *              TP_MLP_ERR_UNSUPPORTED.
 *   Empty      N = 0 tokens (rows = 0, n = 0) is valid.  A buffer whose size
 *              is then zero may be NULL (the storage of an empty tensor);
 *              the weights, gamma and the gradient outputs may not.  A
 *              forward or a reduction launches nothing.  A weight
 *              gradient, db2, dgamma or dbeta, being a sum over the batch's
 *              rows, is written as zeros.  No workspace is needed.
 *   Ownership  The caller allocates and owns every buffer.  The library never
 *              allocates, frees or keeps a pointer after returning.
 *   Streams    All work is enqueued on `stream` (0 = the null stream) and is
 *              never synchronised; inputs must stay valid until the stream
 *              has passed the work.  Asynchronous faults surface at the
 *              caller's next synchronisation.  The library launches only
 *              kernels (no memset, copy, allocation or synchronisation), so
 *              its calls can be captured into a HIP graph on `stream`.
 *   Outputs    Overwritten, never accumulated into.
 *   Errors     Arguments are validated on the host before any launch; an
 *              invalid call returns TP_MLP_ERR_INVALID_ARG (a valid but
 *              unsupported one TP_MLP_ERR_UNSUPPORTED, a missing or short
 *              workspace TP_MLP_ERR_WORKSPACE) and enqueues nothing.  A failed launch returns TP_MLP_ERR_HIP.  Nothing is
 *              printed and no C++ exception crosses the ABI.
 *   Threads    Entry points are reentrant; the only process-wide state is a
 *              once-initialised per-device property cache.
 */
#ifndef TP_MLP_H
#define TP_MLP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TP_MLP_OK = 0,
  TP_MLP_ERR_INVALID_ARG = 1, /* bad pointer, shape, alignment, rank or act */
  TP_MLP_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. t > 64)   */
  TP_MLP_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than required   */
  TP_MLP_ERR_HIP = 4          /* a HIP launch or query failed              */
} tp_mlp_status;

/* Elementwise activation on the rank's hidden columns.
 * RELU:   A = max(U, 0); derivative [U > 0] (0 at U == 0).
 * GELU:   exact erf form, A = U * Phi(U); derivative Phi(U) + U * phi(U).
 * SWIGLU: A = SiLU(G) * U with G = X @ Wg_i (gate) and U = X @ W1_i (up),
 *         SiLU(z) = z * sigmoid(z); gate and up hold the same columns. */
typedef enum {
  TP_MLP_ACT_RELU = 0,
  TP_MLP_ACT_GELU = 1,
  TP_MLP_ACT_SWIGLU = 2
} tp_mlp_act;

/* The problem as the pages state it: replicated input X [N, h], the full
 * intermediate width F split over t ranks, this shard's rank (it owns the
 * contiguous hidden columns [rank*F/t, (rank+1)*F/t), rank 0 lowest), and the
 * activation.  Requires N >= 0, h >= 8, F % t == 0, 1 <= t <= 64,
 * 0 <= rank < t, h % 8 == 0 and (F / t) % 8 == 0. */
typedef struct {
  int64_t n_tokens; /* N = b * s                                   */
  int64_t hidden;   /* h                                           */
  int64_t ffn;      /* F, the full intermediate width (all ranks)  */
  int32_t t;        /* tensor-parallel degree                      */
  int32_t rank;     /* this shard's rank                           */
  int32_t act;      /* tp_mlp_act                                  */
} tp_mlp_shape;

/* ------------------------------------------------------------------------
 * Composite entry points (one call per direction per rank)
 * ------------------------------------------------------------------------ */

/* Forward of one rank's shard ("02 -- Tensor Parallelism", "The MLP
 * pairing"): U_i = X @ W1_i (SwiGLU: also G_i = X @ Wg_i), A_i = act(...),
 * Y_i = A_i @ W2_i, the full-shape PARTIAL sum with no bias.  The ranks'
 * partials are summed (and the bias added) by tp_mlp_reduce_partials_local.
 *   X    bf16 [N, h]        replicated input
 *   W1_i bf16 [h, F_i]      column shard of W1 (= W_up for SwiGLU)
 *   Wg_i bf16 [h, F_i]      column shard of W_gate; non-NULL iff SWIGLU
 *   W2_i bf16 [F_i, h]      row shard of W2 (= W_down)
 *   Y_i  bf16 [N, h]        out: partial sum
 *   A_i  bf16 [N, F_i]      out: activation (input of the backward)
 *   U_i  bf16 [N, F_i]      out or NULL: pre-activation (SwiGLU: up
 *                           projection) stash for the backward
 *   G_i  bf16 [N, F_i]      out or NULL: SwiGLU gate stash; must be NULL
 *                           unless SWIGLU, and given iff U_i is given
 * Three regimes, picked by N:
 *   N == 1       one-token decode: split-K GEMVs that read each weight once
 *                (HBM bound), float32 k-split partials in the workspace;
 *   2 <= N <= 128 small batches: split-K MFMA products that also read
 *                each weight once, float32 k-split partials in the workspace
 *                ("02 -- Tensor Parallelism": decode batches stay memory
 *                bound; up to 128 tokens this is also 2.2-2.6x faster than
 *                the wide tiles, whose 128-row tiles leave most CUs idle);
 *   N > 128      the wide-tile MFMA GEMMs, which need no workspace.
 * All three produce the same quantities to the same tolerance.  workspace:
 * device memory of at least tp_mlp_workspace_bytes(s, 0) bytes, no initial
 * contents required; NULL is allowed when that size is 0.  Calls that share
 * one workspace must be ordered on one stream.  The workspace size depends
 * on the shape only. */
tp_mlp_status tp_mlp_fwd_shard(const tp_mlp_shape* s, const void* X,
                               const void* W1_i, const void* Wg_i,
                               const void* W2_i, void* Y_i, void* A_i,
                               void* U_i, void* G_i, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight decode/serving loops, harnesses that forbid allocation):
 * tp_mlp_fwd_shard with the same arguments, results and kernels (bitwise the
 * same outputs), but no workspace argument.  The k-split partials of the
 * one-token and small-batch paths (1 <= N <= 128) live in a fixed 64 MiB
 * array of device memory inside the library, one per GPU, held until the
 * process ends; this call allocates nothing (no hipMalloc, no allocating
 * library routine).  A shape whose partials need more than 64 MiB returns
 * TP_MLP_ERR_WORKSPACE before any launch (tp_mlp_workspace_bytes(s, 0) gives
 * the need; about 0.5 MiB per token at the 70B shard).  N > 128 takes the
 * wide-tile path, which uses no scratch.  Every call on one GPU shares that
 * GPU's array, so calls that may overlap in time on one GPU (different
 * streams, or concurrent graphs) race on it: order them on one stream.  The
 * array needs no initial contents and its contents between calls are
 * meaningless.  TP_MLP_ERR_HIP if the array's device address cannot be
 * queried on the current device. */
tp_mlp_status tp_mlp_fwd_shard_noalloc(const tp_mlp_shape* s, const void* X,
                                       const void* W1_i, const void* Wg_i,
                                       const void* W2_i, void* Y_i, void* A_i,
                                       void* U_i, void* G_i,
                                       hipStream_t stream);

/* Backward of one rank's shard ("Parallelism Strategies #1 - Tensor
 * Parallelism", sharded backward, in math layout).  dY is the same on every
 * rank (g's backward is the identity).
 *   dA_i = dY @ W2_i^T, then through the activation:
 *     RELU/GELU: dU_i = dA_i * act'(U_i)               -> dU  bf16 [N, F_i]
 *     SWIGLU:    dG = dA*U*s*(1+G*(1-s)), dP = dA*SiLU(G), s = sigmoid(G)
 *                                                     -> dU  bf16 [N, 2*F_i]
 *                laid out as [dG | dP] (columns [0,F_i) then [F_i,2F_i)).
 *   dW2_i = A_i^T @ dY                                 -> fp32 [F_i, h]
 *   dW1_i = X^T @ dU_i (SWIGLU: X^T @ dP = dW_up)     -> fp32 [h, F_i]
 *   dWg_i = X^T @ dG (SWIGLU only; else must be NULL) -> fp32 [h, F_i]
 *   dX_partial = dU_i @ W1_i^T (SWIGLU: dG @ Wg_i^T + dP @ W1_i^T, one
 *     product over K = 2*F_i)                          -> bf16 [N, h]
 *     The ranks' dX_partial must be summed (f's backward); use
 *     tp_mlp_reduce_partials_local with bias NULL.
 *   db2 = sum over rows of dY -> fp32 [h], or NULL to skip.  The output bias
 *     is added once, so pass db2 on one rank only.
 * With 1 <= N <= 128 tokens the two input gradients (dU_i, dX_partial) run
 * as split-K products whose float32 partials are kept in dW2_i and dW1_i
 * before those are written (as tp_mlp_down_bwd_shard and
 * tp_mlp_up_bwd_shard do), and when the two weight gradients' tiles would
 * not fill the GPU even once they then share one launch (the same bits as
 * the step calls); otherwise on the wide tiles.
 * Inputs A_i, U_i (and G_i for SwiGLU) are the forward's outputs; U_i is
 * required.  The products need no workspace; db2 != NULL needs
 * tp_mlp_workspace_bytes(s, 1) bytes of device scratch (no initial contents
 * required).  With db2 == NULL, workspace may be NULL. */
tp_mlp_status tp_mlp_bwd_shard(const tp_mlp_shape* s, const void* X,
                               const void* W1_i, const void* Wg_i,
                               const void* W2_i, const void* dY,
                               const void* A_i, const void* U_i,
                               const void* G_i, void* dU_i, float* dW1_i,
                               float* dWg_i, float* dW2_i, void* dX_partial,
                               float* db2, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* Local stand-in for the all-reduce of g's forward and f's backward ("Tensor
 * and sequence parallelism", table of f and g; "Tensor Parallelism's
 * Communication Boundary" on adding the bias once):
 *   out[r][c] = bf16( (sum_{k=0}^{t-1} float(partials[k][r][c])) + bias[c] )
 * summed in float32 in rank order, the bias (if non-NULL) added once after
 * the sum, one final rounding.
 *   partials  HOST array of t DEVICE pointers, each bf16 [rows, cols]
 *   bias      bf16 [cols] or NULL
 *   out       bf16 [rows, cols]; may coincide exactly with any partials[k]
 *             (each output chunk is written after its inputs are read); any
 *             other overlap with a partial is rejected (INVALID_ARG).
 * Requires 1 <= t <= 64 (t > 64: UNSUPPORTED), rows >= 0, cols % 8 == 0,
 * 16-byte alignment. */
tp_mlp_status tp_mlp_reduce_partials_local(int32_t t,
                                           const void* const* partials,
                                           int64_t rows, int64_t cols,
                                           const void* bias, void* out,
                                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * Sequence-parallel boundary ("Tensor and sequence parallelism", section
 * "Sequence parallelism").  Outside the tensor-parallel region the token rows
 * are split into t contiguous blocks, rank r holding rows
 * [r*rows/t, (r+1)*rows/t).  Leaving the region, the partial sums are added
 * and split back into those blocks (a reduce-scatter); entering it, the
 * blocks are concatenated (an all-gather).  Together they move the same data
 * as the all-reduce they replace.  These are the local stand-ins: all t
 * inputs are on this GPU.
 * ------------------------------------------------------------------------ */

/* Leaving the region (and the backward of entering it, for the partial input
 * gradients): rank `rank`'s block of the reduced sum, with the output bias
 * added once and the residual branch of that block fused in:
 *   out[i][c] = bf16( sum_{k<t} float(partials[k][rank*rows/t + i][c])
 *                     + bias[c] + residual[i][c] )
 * summed in float32 in rank order, then the bias, then the residual, one
 * rounding.
 *   partials  HOST array of t DEVICE pointers, each bf16 [rows, cols]
 *   rank      0 <= rank < t; rows % t == 0
 *   bias      bf16 [cols] or NULL
 *   residual  bf16 [rows/t, cols] or NULL
 *   out       bf16 [rows/t, cols]; may coincide exactly with the residual or
 *             with rank's block of any partials[k]; other overlap with an
 *             input is rejected (INVALID_ARG).
 * Requires 1 <= t <= 64 (t > 64: UNSUPPORTED), cols % 8 == 0, 16-byte
 * alignment. */
tp_mlp_status tp_mlp_reduce_scatter_local(int32_t t,
                                          const void* const* partials,
                                          int64_t rows, int64_t cols,
                                          int32_t rank, const void* bias,
                                          const void* residual, void* out,
                                          hipStream_t stream);

/* Entering the region (and the backward of leaving it, for the output
 * gradient): the t blocks stacked in rank order,
 *   out[r*shard_rows + i][c] = shards[r][i][c]   (a bitwise copy).
 *   shards  HOST array of t DEVICE pointers, each bf16 [shard_rows, cols]
 *   out     bf16 [t*shard_rows, cols]; must not overlap any shard
 *           (INVALID_ARG).
 * Requires 1 <= t <= 64 (t > 64: UNSUPPORTED), shard_rows >= 0,
 * cols % 8 == 0, 16-byte alignment. */
tp_mlp_status tp_mlp_all_gather_local(int32_t t, const void* const* shards,
                                      int64_t shard_rows, int64_t cols,
                                      void* out, hipStream_t stream);

/* Workspace bytes needed by tp_mlp_fwd_shard (backward = 0) or
 * tp_mlp_bwd_shard (backward = 1) for shape s; 0 means none.  Returns 0 for
 * an invalid shape. */
size_t tp_mlp_workspace_bytes(const tp_mlp_shape* s, int backward);

/* Static, NUL-terminated description of a status code. */
const char* tp_mlp_status_string(tp_mlp_status st);

/* ------------------------------------------------------------------------
 * Step-level entry points: the column-parallel and row-parallel pieces the
 * composite calls are made of, one GPU kernel each, on the same shapes and
 * buffers as above.  They exist for callers that schedule the pieces
 * themselves (e.g. to put a collective between them) and for per-kernel
 * timing.
 * ------------------------------------------------------------------------ */

/* Column-parallel up-projection with the activation fused in its epilogue:
 * A_i = act(X @ W1_i) (SwiGLU: SiLU(X @ Wg_i) * (X @ W1_i)), stashing U_i /
 * G_i when non-NULL.  MFMA path for every N (no decode dispatch). */
tp_mlp_status tp_mlp_up_act_shard(const tp_mlp_shape* s, const void* X,
                                  const void* W1_i, const void* Wg_i,
                                  void* A_i, void* U_i, void* G_i,
                                  hipStream_t stream);

/* Row-parallel down-projection: Y_i = A_i @ W2_i (partial sum, no bias). */
tp_mlp_status tp_mlp_down_shard(const tp_mlp_shape* s, const void* A_i,
                                const void* W2_i, void* Y_i,
                                hipStream_t stream);

/* dgrad through W2 fused with the activation derivative:
 * dU_i = (dY @ W2_i^T) * act'(U_i) (SwiGLU: [dG | dP] from G_i, U_i). */
tp_mlp_status tp_mlp_down_dgrad_act_shard(const tp_mlp_shape* s,
                                          const void* dY, const void* W2_i,
                                          const void* U_i, const void* G_i,
                                          void* dU_i, hipStream_t stream);

/* wgrad of W2: dW2_i = A_i^T @ dY (fp32). */
tp_mlp_status tp_mlp_down_wgrad_shard(const tp_mlp_shape* s, const void* A_i,
                                      const void* dY, float* dW2_i,
                                      hipStream_t stream);

/* wgrad of W1 (and W_gate): dW1_i = X^T @ dU_i (SwiGLU: dWg_i = X^T @ dG,
 * dW1_i = X^T @ dP) (fp32). */
tp_mlp_status tp_mlp_up_wgrad_shard(const tp_mlp_shape* s, const void* X,
                                    const void* dU_i, float* dW1_i,
                                    float* dWg_i, hipStream_t stream);

/* Both weight gradients in one launch (what tp_mlp_bwd_shard runs): dW2_i
 * as tp_mlp_down_wgrad_shard and dW1_i (dWg_i) as tp_mlp_up_wgrad_shard,
 * their tiles sharing the waves of blocks so that neither leaves a partial
 * last wave on its own.  Each element is summed over the tokens in the same
 * order as in the separate calls: the results are bitwise the same. */
tp_mlp_status tp_mlp_wgrad_shard(const tp_mlp_shape* s, const void* X,
                                 const void* A_i, const void* dY,
                                 const void* dU_i, float* dW1_i, float* dWg_i,
                                 float* dW2_i, hipStream_t stream);

/* dgrad through W1: dX_partial = dU_i @ W1_i^T (SwiGLU: [dG | dP] @
 * [Wg_i | W1_i]^T). */
tp_mlp_status tp_mlp_up_dgrad_shard(const tp_mlp_shape* s, const void* dU_i,
                                    const void* W1_i, const void* Wg_i,
                                    void* dX_partial, hipStream_t stream);

/* The down-projection's backward, the first half of what tp_mlp_bwd_shard
 * runs: dU_i as tp_mlp_down_dgrad_act_shard and dW2_i = A_i^T @ dY as
 * tp_mlp_down_wgrad_shard.  Both need only the forward's outputs and dY, so
 * they share one launch when their block tiles fill the GPU at least once
 * (the tiles of the longer product are dispatched first, the other's fill
 * in behind them); otherwise they run one after the other.  Each element is
 * summed in the same order either way: the results are bitwise those of the
 * separate calls.  Exception, 1 <= N <= 128 with h >= N: dU_i runs as a
 * split-K product (the few token rows leave the wide tiles' grid nearly
 * empty) whose float32 partials are kept in dW2_i before dW2_i is computed;
 * dW2_i is still bitwise that of the separate call, dU_i equal to it up to
 * the order of its float32 sums.  N = 0: dW2_i is written as zeros. */
tp_mlp_status tp_mlp_down_bwd_shard(const tp_mlp_shape* s, const void* dY,
                                    const void* W2_i, const void* U_i,
                                    const void* G_i, const void* A_i,
                                    void* dU_i, float* dW2_i,
                                    hipStream_t stream);

/* The up-projection's backward, the second half of what tp_mlp_bwd_shard
 * runs: dX_partial as tp_mlp_up_dgrad_shard and dW1_i (dWg_i) as
 * tp_mlp_up_wgrad_shard, both from dU_i, in one launch or two as for
 * tp_mlp_down_bwd_shard, bitwise equal to the separate calls.  Exception,
 * 1 <= N <= 128 with F_i >= g*N (g = 2 for SwiGLU, else 1): dX_partial runs
 * as a split-K product whose partials are kept in dW1_i first, equal to the
 * separate call up to the order of its float32 sums.  N = 0: the weight
 * gradients are written as zeros. */
tp_mlp_status tp_mlp_up_bwd_shard(const tp_mlp_shape* s, const void* X,
                                  const void* dU_i, const void* W1_i,
                                  const void* Wg_i, void* dX_partial,
                                  float* dW1_i, float* dWg_i,
                                  hipStream_t stream);

/* db2 = column sums of dY [rows, cols] (fp32 out [cols]): the gradient of the
 * output bias that is added once after the reduction.  Deterministic
 * (fixed-order float32 sums).  workspace: device scratch of at least
 * tp_mlp_bias_grad_workspace_bytes(rows, cols) bytes, no initial contents
 * required (none when rows = 0: db2 is then zero).  Requires rows >= 0,
 * cols % 8 == 0. */
tp_mlp_status tp_mlp_bias_grad(const void* dY, int64_t rows, int64_t cols,
                               float* db2, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);
size_t tp_mlp_bias_grad_workspace_bytes(int64_t rows, int64_t cols);

/* ------------------------------------------------------------------------
 * Attention block projections ("02 -- Tensor Parallelism", section "The
 * attention pairing"; "Megatron-LM: Tensor Parallelism", section "Attention
 * Block"; "Tensor and sequence parallelism", closing exercise 1).  The same
 * pairing as the MLP: the Q, K and V projections are column-parallel by head,
 * the output projection row-parallel into a full-shape partial sum.  The
 * attention core between them (scores, softmax, weighted sum) is not part of
 * this library: the caller passes its output O_i and, backward, its
 * gradient dQKV_i.
 *
 * Heads: rank r owns query heads [r*n_heads/t, (r+1)*n_heads/t) and the
 * key/value heads of their groups (query head j is in group
 * j / (n_heads / n_kv_heads)): the block [r*n_kv/t, (r+1)*n_kv/t) when
 * n_kv_heads >= t, else the single head r*n_kv/t, which is then replicated
 * on t/n_kv_heads ranks (its weight gradients must be summed over those
 * replicas).  Head j owns head_dim consecutive columns.  Requires
 * n_heads % n_kv_heads == 0, n_heads % t == 0, n_kv_heads % t == 0 or
 * t % n_kv_heads == 0, head_dim % 8 == 0, hidden % 8 == 0, 1 <= t <= 64.
 *
 * Widths on rank r: qc = n_heads/t * head_dim; kvc = (n_kv/t or 1) *
 * head_dim; qkvc = qc + 2*kvc.  Buffers (bf16 unless noted, row-major):
 *   X       [N, h]        replicated input
 *   Wqkv_i  [h, qkvc]     [W_q columns of its query heads | W_k columns of
 *                         its key/value heads | W_v columns of the same]
 *   QKV_i   [N, qkvc]     out: [Q_i | K_i | V_i]
 *   O_i     [N, qc]       the attention core's output for the rank's heads
 *   Wo_i    [qc, h]       the W_o rows of the rank's query heads
 *   Y_i     [N, h]        out: partial sum (add over ranks; bias once after)
 * ------------------------------------------------------------------------ */
typedef struct {
  int64_t n_tokens;   /* N                                      */
  int64_t hidden;     /* h                                      */
  int32_t n_heads;    /* query heads                            */
  int32_t n_kv_heads; /* key/value heads (= n_heads without GQA) */
  int32_t head_dim;
  int32_t t;          /* tensor-parallel degree                 */
  int32_t rank;
} tp_attn_shape;

/* Workspace bytes the forward projections need for shape s: nonzero only
 * when 1 <= n_tokens <= 128, where tp_attn_qkv_shard and tp_attn_out_shard
 * take the small-batch path (split-K products that stream each weight once,
 * then a fixed-order sum of the k-splits, the arithmetic of the MLP's
 * small-batch path); 0 for larger N or an invalid shape. */
size_t tp_attn_workspace_bytes(const tp_attn_shape* s);

/* Column-parallel QKV projection: QKV_i = X @ Wqkv_i (no communication).
 *   workspace  tp_attn_workspace_bytes(s) bytes of device scratch (no
 *              initial contents needed; NULL when that is 0); missing or
 *              smaller: TP_MLP_ERR_WORKSPACE. */
tp_mlp_status tp_attn_qkv_shard(const tp_attn_shape* s, const void* X,
                                const void* Wqkv_i, void* QKV_i,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Row-parallel output projection: Y_i = O_i @ Wo_i, the full-shape partial
 * sum (sum over ranks with tp_mlp_reduce_partials_local, bias once).
 *   workspace  as for tp_attn_qkv_shard. */
tp_mlp_status tp_attn_out_shard(const tp_attn_shape* s, const void* O_i,
                                const void* Wo_i, void* Y_i,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Backward of the output projection for dY [N, h] (the same on every rank):
 *   dO_i  = dY @ Wo_i^T  -> bf16 [N, qc]  (input of the attention core's
 *                                          backward)
 *   dWo_i = O_i^T @ dY   -> fp32 [qc, h]
 * With 1 <= N <= 128 tokens (and h >= N) dO_i runs as the small-batch
 * split-K product, whose float32 partials are kept in dWo_i before dWo_i is
 * computed, as long as those partials (written and read back) stay within
 * Wo_i's bytes; otherwise on the wide tiles, split along k the same way when
 * their grid leaves most CUs idle. */
tp_mlp_status tp_attn_out_bwd_shard(const tp_attn_shape* s, const void* dY,
                                    const void* O_i, const void* Wo_i,
                                    void* dO_i, float* dWo_i,
                                    hipStream_t stream);

/* Backward of the QKV projection for dQKV_i [N, qkvc] (the attention core's
 * gradient, laid out like QKV_i):
 *   dX_partial = dQKV_i @ Wqkv_i^T -> bf16 [N, h]  (sum over ranks)
 *   dWqkv_i    = X^T @ dQKV_i      -> fp32 [h, qkvc]
 * With 1 <= N <= 128 tokens (and qkvc >= N) dX_partial runs as the
 * small-batch split-K product with its partials in dWqkv_i, then dWqkv_i, as
 * long as those partials stay within Wqkv_i's bytes (as for dO_i). */
tp_mlp_status tp_attn_qkv_bwd_shard(const tp_attn_shape* s, const void* X,
                                    const void* Wqkv_i, const void* dQKV_i,
                                    float* dWqkv_i, void* dX_partial,
                                    hipStream_t stream);

/* The same backward split for callers that schedule the output
 * projection's weight gradient late: the attention core's backward needs
 * only dO_i, and dWo_i = O_i^T @ dY can wait to share a launch with the QKV
 * projection's backward (both are weight gradients over the tokens).
 *
 * dO_i = dY @ Wo_i^T -> bf16 [N, qc], alone.  With 1 <= N <= 128 tokens, or
 * when its tile grid would leave most CUs idle, it runs split along k into
 * float32 partials in the workspace, summed in slice order and rounded once
 * (the same splits and arithmetic as tp_attn_out_bwd_shard's dO_i, which
 * borrows dWo_i's storage instead: the same bits).
 *   workspace  tp_attn_out_dgrad_workspace_bytes(s) bytes of device scratch
 *              (no initial contents needed; NULL when that is 0); missing or
 *              smaller: TP_MLP_ERR_WORKSPACE. */
size_t tp_attn_out_dgrad_workspace_bytes(const tp_attn_shape* s);
tp_mlp_status tp_attn_out_dgrad_shard(const tp_attn_shape* s, const void* dY,
                                      const void* Wo_i, void* dO_i,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* tp_attn_qkv_bwd_shard's dX_partial and dWqkv_i together with the output
 * projection's deferred dWo_i = O_i^T @ dY (fp32 [qc, h]), in one launch when
 * the block tiles fill the GPU (dX_partial's tiles first, the two weight
 * gradients' filling in behind them), else one after the other (with
 * 1 <= N <= 128 tokens: dX_partial as in tp_attn_qkv_bwd_shard, then both
 * weight gradients in one launch).  Each element is summed in the same order
 * as in the separate calls: the results are bitwise theirs. */
tp_mlp_status tp_attn_qkv_bwd_out_wgrad_shard(const tp_attn_shape* s,
                                              const void* X,
                                              const void* Wqkv_i,
                                              const void* dQKV_i,
                                              const void* dY,
                                              const void* O_i,
                                              float* dWqkv_i,
                                              void* dX_partial,
                                              float* dWo_i,
                                              hipStream_t stream);

/* ------------------------------------------------------------------------
 * LayerNorm of the sequence-parallel region ("Tensor and sequence
 * parallelism", section "Sequence parallelism" and its check script;
 * "02 -- Tensor Parallelism", the paragraph on LayerNorm and dropout between
 * the two all-reduces).  Under sequence parallelism the LayerNorm works on
 * the rank's own block of rows/t token rows; its output enters the
 * tensor-parallel region through the all-gather, and the LayerNorm weights,
 * shared by every block, have their gradients summed over the group.
 *
 * Per row of length h = cols:
 *   mean = sum(x)/h,  var = sum((x - mean)^2)/h (biased),
 *   rstd = 1/sqrt(var + eps),  y = (x - mean)*rstd*gamma + beta,
 * computed in float32 from the bf16 row (mean and the centred variance from
 * registers, two passes), y rounded to bf16 once.  Row statistics and the
 * weight-gradient column sums are added in a fixed order: results are
 * deterministic.  Dropout is not part of this path (probability 0).
 *
 * Common requirements: rows >= 0, 8 <= cols <= 16384 (larger: UNSUPPORTED),
 * cols % 8 == 0, eps > 0 and finite, every pointer a 16-byte aligned device
 * pointer.
 * ------------------------------------------------------------------------ */

/* y = LayerNorm(x).
 *   x          bf16 [rows, cols]: the rank's block of token rows
 *   gamma      bf16 [cols]; beta bf16 [cols] or NULL (no bias)
 *   y          out bf16 [rows, cols]; may be the rank's block inside the
 *              all-gather destination; may coincide exactly with x, must not
 *              otherwise overlap an input
 *   mean, rstd out float32 [rows] each (the backward's stash), or both NULL
 *              (inference). */
tp_mlp_status tp_sp_layernorm_fwd(int64_t rows, int64_t cols, float eps,
                                  const void* x, const void* gamma,
                                  const void* beta, void* y, float* mean,
                                  float* rstd, hipStream_t stream);

/* Leaving the tensor-parallel region into the next LayerNorm, in one pass:
 * the reduce-scatter of tp_mlp_reduce_scatter_local,
 *   z = bf16( sum_{k<t} partials[k][rank*rows/t + i][c] + bias[c]
 *             + residual[i][c] )                (the new residual stream)
 * then y = LayerNorm(z) of the stored bf16 z, exactly as the two separate
 * calls would compute it.
 *   partials, rows, cols, rank, bias, residual: as for
 *              tp_mlp_reduce_scatter_local (rows % t == 0, 1 <= t <= 64);
 *   z          out bf16 [rows/t, cols]; the same overlap rules as that
 *              call's out;
 *   gamma, beta, y, mean, rstd: as for tp_sp_layernorm_fwd over the
 *              rows/t rows; y must not overlap z or any input. */
tp_mlp_status tp_sp_reduce_scatter_layernorm_local(
    int32_t t, const void* const* partials, int64_t rows, int64_t cols,
    int32_t rank, const void* bias, const void* residual, void* z, float eps,
    const void* gamma, const void* beta, void* y, float* mean, float* rstd,
    hipStream_t stream);

/* Backward of tp_sp_layernorm_fwd for the output gradient dy:
 *   xhat = (x - mean)*rstd,  g = dy*gamma,
 *   dx = rstd*(g - sum(g)/h - xhat*sum(g*xhat)/h) + dres,
 *   dgamma = sum over the rows of dy*xhat,  dbeta = sum over the rows of dy.
 * dgamma and dbeta cover this block's rows only: the group's gradient is
 * their sum over the ranks (tp_sp_sum_grads_local).
 *   x          bf16 [rows, cols]: the forward's input
 *   gamma      bf16 [cols]
 *   mean, rstd float32 [rows]: the forward's stash
 *   dy         bf16 [rows, cols]
 *   dres       bf16 [rows, cols] or NULL: the gradient arriving along the
 *              residual branch, added to dx
 *   dx         out bf16 [rows, cols]; may coincide exactly with dy or dres,
 *              must not otherwise overlap an input
 *   dgamma     out float32 [cols]; dbeta out float32 [cols] or NULL
 *   workspace  tp_sp_layernorm_bwd_workspace_bytes(rows, cols) bytes of
 *              device scratch (no initial contents needed; smaller:
 *              TP_MLP_ERR_WORKSPACE). */
tp_mlp_status tp_sp_layernorm_bwd(int64_t rows, int64_t cols, const void* x,
                                  const void* gamma, const float* mean,
                                  const float* rstd, const void* dy,
                                  const void* dres, void* dx, float* dgamma,
                                  float* dbeta, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes for tp_sp_layernorm_bwd; 0 for invalid sizes. */
size_t tp_sp_layernorm_bwd_workspace_bytes(int64_t rows, int64_t cols);

/* The all-reduce of a parameter shared by the sequence blocks (the LayerNorm
 * weight and bias): out[i] = sum_{k<t} grads[k][i], float32, rank order.
 *   grads  HOST array of t DEVICE pointers, each float32 [n]
 *   out    float32 [n]; may coincide exactly with grads[0] (any rank's
 *          buffer would be read after it is written), must not otherwise
 *          overlap an input.
 * Requires 1 <= t <= 64 (t > 64: UNSUPPORTED), n >= 0, n % 4 == 0. */
tp_mlp_status tp_sp_sum_grads_local(int32_t t, const float* const* grads,
                                    int64_t n, float* out,
                                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TP_MLP_H */
