/*
 * lion_attn.h -- C ABI of the LION bidirectional masked linear attention library for AMD
 * Instinct MI355X (gfx950).
 *
 * For every batch b and head h the library computes, from queries q, keys k and values v,
 *
 *     y_i = sum_j M_ij (phi(q_i) . phi(k_j)) v_j / ( sum_j M_ij (phi(q_i) . phi(k_j)) + eps )
 *
 * that is Y = SCALE(phi(Q) phi(K)^T (.) M) V with SCALE the row normalisation.  The mask M holds
 * the products of per-token decays lambda between positions i and j, in either direction:
 * M_ii = 1 and, for i < j, M_ij = M_ji = lambda_{i+1} * ... * lambda_j.
 *
 * Sources, all on the page "LION: A bidirectional framework that trains like a Transformer and
 * infers like an RNN" (author-reviewer discussion) unless said otherwise:
 *   - attention form Y = SCALE(QK^T (.) M)V and its equivalent bidirectional RNN: reply
 *     "Concern 1", Theorem 3.3 Eq. 25 and Eq. 20-24;
 *   - the RNN that keeps one vector y and one scalar c per token and direction: reply
 *     "1: Recurrence Form of Linear Attention";
 *   - chunking for parallel inference: reply "4: Practicality of Recurrent Inference", and the
 *     blog page "LION Part IV - Results", section "LION Architecture Variants and Trade-offs";
 *   - the three mask kinds LION-LIT (lambda = 1), LION-RETNET / LION-D (fixed per-head decay) and
 *     LION-S (input-dependent lambda_i): reply "(3) ... two distinct methodological
 *     contributions"; phi = elu()+1 for LIT and normalised silu for S: item 4, "Default
 *     non-linearity".
 *
 * Three entry points compute the same Y by the three forms; results agree up to rounding.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   q, k, v      device pointers, contiguous row-major [B, H, L, d], element type `dtype`.
 *   log_lambda   device pointer to fp32 log(lambda), every entry finite and <= 0:
 *                  LION_MASK_LIT: must be NULL (lambda = 1);
 *                  LION_MASK_D:   [H]        one decay per head;
 *                  LION_MASK_S:   [B, H, L]  one decay per token (entry 0 of each row never enters).
 *   mask_kind    LION_MASK_LIT / LION_MASK_D / LION_MASK_S, optionally | LION_CAUSAL (keys after
 *                the query are masked out) and | LION_FP32_ARITH; the kind also selects phi:
 *                  LIT: phi(x) = elu(x) + 1;  D: phi(x) = x;  S: phi = silu(x) / ||silu(x)||_2 over the
 *                  d channels of the token (an all-zero silu vector gives phi = 0).
 *   eps          >= 0 and finite, added to every row sum.
 *   B, H, L      >= 1;  d in {16, 32, 64, 128}.
 *   dtype        LION_DTYPE_BF16 or LION_DTYPE_F32: element type of q, k, v.
 *   y            device pointer, contiguous [B, H, L, d], element type `y_dtype`;
 *                y_dtype is dtype, or LION_DTYPE_F32 when dtype is bf16 (an fp32 output keeps
 *                the kernel's fp32 result unrounded).
 *   den_out      NULL, or device pointer to fp32 [B, H, L] receiving each row sum + eps.
 *   stream       a hipStream_t; NULL means the default stream.
 * Every device pointer must be 16-byte aligned.
 *
 * Precision: bf16 inputs feed bf16 matrix-core products with fp32 accumulation; phi and the
 * row-sum products are formed in fp32 and rounded to bf16 before the products that need them.
 * fp32 inputs, and bf16 inputs with LION_FP32_ARITH, keep every step in fp32.  Row sums (denominators)
 * are accumulated in fp32.
 *
 * Ownership and threading: the caller allocates and owns every buffer, workspace included.  The
 * library allocates and frees nothing, never synchronises, and is reentrant; its one piece of global
 * state is the scratch array of lion_attn_chunk_noalloc (one copy per GPU) and that array's per-device
 * address.  All work is enqueued on `stream`; outputs are valid once the stream reaches that
 * point.  Input buffers are only read; y, den_out and the workspace are written.
 *
 * Errors: every entry point returns LION_OK (0) or a negative status.  Argument errors are found
 * on the host before any HIP call and leave every buffer untouched:
 *   LION_ERR_INVALID      a required pointer is NULL or misaligned, a size is out of range, eps is
 *                         negative or not finite, an enum is unknown, or log_lambda is given for LIT
 *                         / missing for D and S;
 *   LION_ERR_UNSUPPORTED  a valid but unimplemented combination (d, C, dtype / y_dtype);
 *   LION_ERR_WORKSPACE    the workspace is smaller than lion_attn_workspace_bytes() asks for;
 *   LION_ERR_HIP          a HIP launch reported an error (hipGetLastError after the launch).
 * Faults inside a kernel surface at the caller's next synchronisation.  No exception crosses the
 * ABI.
 */
#ifndef LION_ATTN_H
#define LION_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LION_ATTN_ABI_VERSION 1

#if defined(__GNUC__)
#define LION_API __attribute__((visibility("default")))
#else
#define LION_API
#endif

enum lion_mask_kind { LION_MASK_LIT = 0, LION_MASK_D = 1, LION_MASK_S = 2 };
/* OR-ed into mask_kind: the causal (unidirectional) variant, M_ij = 0 for j > i -- the forward
 * recurrence S_i = lambda_i S_{i-1} + phi(k_i) v_i^T alone, causal linear attention (reply "1:
 * Recurrence Form of Linear Attention", Eq. 4a-4c) with the kind's decay (LION-S 1D for
 * single-directional generation: reply item 5, "Is this method limited to bidirectional models?"). */
enum { LION_CAUSAL = 4 };
/* OR-ed into mask_kind (full, chunkwise and RNN forms): fp32 arithmetic throughout for bf16 inputs.  The
 * inputs are upcast exactly as they are staged, and phi, the scores, the masked scores, the carried
 * states and the products run in fp32 (fp32 matrix cores), as for fp32 inputs, instead of being rounded
 * to bf16 for the bf16 matrix cores.  For rows whose denominator nearly cancels (LION-S with normalised
 * silu: condition numbers in the thousands), where bf16 rounding is amplified by the condition number;
 * pair it with an fp32 y.  Slower (fp32 matrix-core peak is 1/16 of bf16).  The RNN form computes in fp32
 * already and ignores it; the two-order and backward entry points return LION_ERR_UNSUPPORTED. */
enum { LION_FP32_ARITH = 8 };
enum lion_dtype { LION_DTYPE_F32 = 0, LION_DTYPE_BF16 = 1 };
enum lion_form { LION_FORM_FULL = 0, LION_FORM_CHUNK = 1, LION_FORM_BIRNN = 2, LION_FORM_FULL_BWD = 3,
                 LION_FORM_CHUNK_BWD = 4, LION_FORM_CHUNK2 = 5 };
enum lion_status {
    LION_OK = 0,
    LION_ERR_INVALID = -1,
    LION_ERR_UNSUPPORTED = -2,
    LION_ERR_WORKSPACE = -3,
    LION_ERR_HIP = -4
};

/* Full (attention) form: the L x L masked score matrix is formed tile by tile on chip and never
 * written out; the mask is generated from prefix sums of log(lambda) inside the kernel.
 * Source: Theorem 3.3 Eq. 25, reply "Concern 1" (the form LION trains with).
 * Needs no workspace. */
LION_API int lion_attn_full(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind, float eps,
                   int B, int H, int L, int d, int dtype, void *y, int y_dtype, float *den_out, void *stream);

/* Full form with the average of two masks, M = (M_b + M_c) / 2: M_b along the tokens' own order and
 * M_c the same product-of-decays mask along a second order of the same tokens, each token keeping its
 * own decay -- the patch-reordered vision models (LION-D and LION-S with "natural" patch orders) average
 * the masks of two patch orders (reply "P2: Comparison against vision SSMs", item 1, Figure 7 b and c).
 *   order   device int32 [L]: order[p] = the token at position p of the second order; must be a
 *           permutation of 0 .. L-1 (not checked on the device: other contents give unspecified
 *           results, never an out-of-bounds access).  For an image the column-major raster of the patch
 *           grid (the class token first).
 *   mask_kind  LIT, D or S; LION_CAUSAL is LION_ERR_UNSUPPORTED.  LIT's mask is all ones in any order.
 * Other arguments as lion_attn_full; no workspace. */
LION_API int lion_attn_full2(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind,
                             float eps, const int *order, int B, int H, int L, int d, int dtype, void *y,
                             int y_dtype, float *den_out, void *stream);

/* Chunkwise form: masked attention inside chunks of C consecutive tokens plus forward and
 * backward d x (d+1) states carried from chunk to chunk.  C in {16, 32, 64, 128, 256} (at most 128
 * when d = 128; larger is LION_ERR_UNSUPPORTED); the last chunk may be partial.  Source: reply "4: Practicality of Recurrent Inference"; blog "LION Part
 * IV - Results", "LION Chunk".
 * workspace: device buffer of at least lion_attn_workspace_bytes(LION_FORM_CHUNK, ...) bytes
 * (may be NULL when that is 0); its contents on entry do not matter and on exit are unspecified. */
LION_API int lion_attn_chunk(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind, int C,
                    float eps, int B, int H, int L, int d, int dtype, void *y, int y_dtype, float *den_out,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Chunkwise form with the two-order averaged mask of lion_attn_full2 (same definition, same order
 * argument; reply "P2: Comparison against vision SSMs", item 1, Figure 7 b and c).  The attention is
 * linear in the mask, so this runs the chunkwise form in the tokens' own order and in the second
 * order (q, k, v and LION-S's log(lambda) rearranged into it in the workspace) with fp32 results and
 * combines y = (y_b den_b + y_c den_c) / (den_b + den_c).
 *   order      device int32 [L], as for lion_attn_full2.
 *   C          as for lion_attn_chunk.  LION_CAUSAL is LION_ERR_UNSUPPORTED.
 *   workspace  >= lion_attn_workspace_bytes(LION_FORM_CHUNK2, ..., C, dtype) bytes: the rearranged
 *              inputs, two fp32 outputs and row sums, and the chunkwise form's own workspace.
 * den_out, when given, receives the averaged mask's row sums + eps (as lion_attn_full2's). */
LION_API int lion_attn_chunk2(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind,
                              int C, float eps, const int *order, int B, int H, int L, int d, int dtype, void *y,
                              int y_dtype, float *den_out, void *workspace, size_t workspace_bytes, void *stream);

/* Chunkwise form without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation).  Same arguments,
 * kernels and results as lion_attn_chunk; the scratch lion_attn_chunk would take from the caller's
 * workspace comes instead from a file-scope device array of LION_NOALLOC_SCRATCH_BYTES held by each GPU
 * the library runs on until the process ends.  The call allocates and frees nothing (its first call on
 * a device looks up that device's copy of the array).
 *   Sizes whose workspace (lion_attn_workspace_bytes(LION_FORM_CHUNK, ...)) exceeds
 *   LION_NOALLOC_SCRATCH_BYTES return LION_ERR_WORKSPACE before any HIP call.
 *   Calls on one GPU share its array: calls that overlap in time on one GPU (other streams, other host
 *   threads) race and give unspecified results; calls ordered on one stream are safe.  The chunkwise
 *   kernels read nothing of the scratch they did not write in the same call.
 * Errors as for lion_attn_chunk; LION_ERR_HIP also when the device copy of the array cannot be found. */
#define LION_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
LION_API int lion_attn_chunk_noalloc(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind,
                                     int C, float eps, int B, int H, int L, int d, int dtype, void *y, int y_dtype,
                                     float *den_out, void *stream);

/* Bidirectional RNN form: a forward and a backward recurrence over tokens with d x d matrix
 * states, S_i = lambda_i S_{i-1} + phi(k_i) v_i^T (backward: S_i = lambda_{i+1} S_{i+1} + ...),
 * keeping only a vector and a scalar per token and direction; the diagonal term is counted once.
 * Source: Theorem 3.3 Eq. 20-24, reply "Concern 1"; reply "1: Recurrence Form of Linear
 * Attention".
 * workspace: as for lion_attn_chunk, sized by lion_attn_workspace_bytes(LION_FORM_BIRNN, ...). */
LION_API int lion_attn_birnn(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind, float eps,
                    int B, int H, int L, int d, int dtype, void *y, int y_dtype, float *den_out, void *workspace,
                    size_t workspace_bytes, void *stream);

/* Backward pass of the full form: the gradients of y = lion_attn_full(q, k, v, log_lambda) for an
 * incoming gradient dy, i.e. dq, dk, dv and d log_lambda.  LION trains with the attention form (the
 * OpenReview title and abstract; Theorem 3.3 Eq. 25, reply "Concern 1"); the pages
 * print no backward formulas, so this is the chain rule of the definition above:
 *   delta_i = dy_i . y_i / den_i,   dp_ij = dy_i . v_j / den_i - delta_i,   dv_j = sum_i M_ij s_ij dy_i / den_i,
 *   dphi(q_i) = sum_j M_ij dp_ij phi(k_j),  dphi(k_j) = sum_i M_ij dp_ij phi(q_i),  then phi's Jacobian;
 *   d log(lambda_u) = sum over pairs (i, j) with min(i,j) < u <= max(i,j) of dp_ij M_ij s_ij
 *   (LION-D: summed over every batch entry and token of the head; LION-S: entry 0 is always 0).
 * q, k, v, log_lambda, mask_kind (LION_CAUSAL allowed), B, H, L, d: as for the forward call.
 *   dtype      must be LION_DTYPE_BF16 (q, k, v, y, dy); fp32 inputs are LION_ERR_UNSUPPORTED.
 *   d          32, 64 or 128 (16 is LION_ERR_UNSUPPORTED).
 *   y, den     the forward call's y (bf16) and den_out (fp32 [B, H, L], row sum + eps) for these inputs.
 *   dy         bf16 [B, H, L, d].
 *   dq, dk, dv written, [B, H, L, d] of type grad_dtype (bf16 or fp32).
 *   dlog_lambda  written: NULL for LIT; fp32 [H] for D; fp32 [B, H, L] for S.
 *   workspace  >= lion_attn_workspace_bytes(LION_FORM_FULL_BWD, ...) bytes (12 B H L); contents on
 *              entry do not matter.
 * Errors as for the forward entry points. */
LION_API int lion_attn_full_bwd(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind,
                                int B, int H, int L, int d, int dtype, const void *y, const float *den,
                                const void *dy, void *dq, void *dk, void *dv, int grad_dtype, float *dlog_lambda,
                                void *workspace, size_t workspace_bytes, void *stream);

/* Backward pass computed the chunkwise way: the same gradients as lion_attn_full_bwd (same formulas),
 * with pairs inside a chunk of C tokens formed directly and the rest of the sequence entering through
 * d x (d+1) states per chunk boundary (the keys' states of the chunkwise forward, and the same
 * construction over phi(q) and [dy / den, -delta]), so the work grows as L C d + L d^2 rather than
 * L^2 d.  Sources: as for lion_attn_full_bwd, and the chunkwise form of lion_attn_chunk (reply
 * "4: Practicality of Recurrent Inference"; blog "LION Part IV - Results", "LION Chunk").
 *   C          16 or 32 (fp32 matrix-core products, fp32 states), 64 or 128 (bf16 matrix-core products
 *              with fp32 sums, as the full form's backward; 128 needs d <= 64); other values are
 *              LION_ERR_UNSUPPORTED.
 *   every other argument as for lion_attn_full_bwd; y and den may come from any forward form.
 *   workspace  >= lion_attn_workspace_bytes(LION_FORM_CHUNK_BWD, ..., C, ...) bytes: four states per
 *              chunk and (batch, head) -- C <= 32: fp32 d x (d+1) (rows padded to d + 4); C >= 64: a
 *              bf16 d x d block and an fp32 last column -- plus 8 B H L; contents on entry do not matter.
 * Errors as for the forward entry points. */
LION_API int lion_attn_chunk_bwd(const void *q, const void *k, const void *v, const float *log_lambda, int mask_kind,
                                 int C, int B, int H, int L, int d, int dtype, const void *y, const float *den,
                                 const void *dy, void *dq, void *dk, void *dv, int grad_dtype, float *dlog_lambda,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* LION-S selectivity prologue: the per-token decays from the layer input, as log(lambda) for the
 * attention entry points, and the key-path input scale of zero-order-hold discretisation.  Sources:
 * lambda_i input-dependent, the scalar version of Mamba-2's state matrix (reply "1. Some
 * equations/notations are not clear enough", Eq. 5a); exp(a_i) on the state and exp(a_i) - 1 on the
 * input (reply "Concern 8").  The pages print neither formula; reading: per head h,
 *   z_i = x_i . w_h + b_h,  log_lambda = a_i = log sigmoid(z_i),  key_scale = exp(a_i) - 1 = -sigmoid(-z_i),
 *   k_out = key_scale * k  (the raw key; pass k_out as the attention's k).
 *   x          bf16 [B, L, Dm], the layer input shared by the heads;  w  bf16 [H, Dm];  bias  fp32 [H].
 *   Dm         a multiple of 32 (else LION_ERR_UNSUPPORTED).
 *   log_lambda written, fp32 [B, H, L].
 *   key_scale  NULL, or written, fp32 [B, H, L].
 *   k, k_out   both NULL, or bf16 [B, H, L, d] with d a multiple of 8 (else LION_ERR_UNSUPPORTED);
 *              k_out may equal k (in place).
 * Device pointers 16-byte aligned; errors as for the attention entry points; no workspace. */
LION_API int lion_selectivity(const void *x, const void *w, const float *bias, int B, int L, int H, int Dm,
                              float *log_lambda, float *key_scale, const void *k, void *k_out, int d, void *stream);

/* Workspace bytes `form` needs for these sizes (C is ignored except for LION_FORM_CHUNK,
 * LION_FORM_CHUNK_BWD and LION_FORM_CHUNK2).
 * Returns 0 when no workspace is needed, and (size_t)-1 for arguments the form rejects. */
LION_API size_t lion_attn_workspace_bytes(int form, int B, int H, int L, int d, int C, int dtype);

/* Static, NUL-terminated description of a status code. */
LION_API const char *lion_status_str(int status);

/* LION_ATTN_ABI_VERSION of the built library. */
LION_API int lion_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LION_ATTN_H */
