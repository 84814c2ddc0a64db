/*
 * mha.h - C ABI of the MI355X (gfx950) multi-head attention forward library.
 *
 * What is computed
 * ----------------
 * Page "Multi-head attention and self-attention", Definition: for query,
 * key and value matrices Q [n_q x d_q], K [n_k x d_k], V [n_k x d_v], head i
 * is scaled dot-product attention of (Q W_i^Q, K W_i^K, V W_i^V) under one
 * mask shared by every head; the heads are concatenated along the feature
 * axis in head order and multiplied by W^O [h*d_vh x d_o].  Self-attention
 * is the case Q = K = V.
 * Page "Stable summary of an attention key block", Definition: the row
 * softmax is computed as running (m, l, z) summaries of key blocks merged
 * with the page's rule, so no score matrix is ever written to memory.
 * Review page "Multi-Head Attention", "Separate and Combined Projections":
 * weights are passed combined, head r occupying a contiguous column block.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor is dense, row-major, with the shapes given below, and lives
 *   in device memory (hipMalloc'd or equivalent) unless a comment says host.
 * - Q, K, V and the weights have element type mha_dims.in_dtype.  The
 *   intermediates of mha_forward (projected heads, the softmax weights fed
 *   to the value product, the concatenated heads) have element type
 *   mha_dims.work_dtype, rounded to nearest even; every sum is accumulated
 *   in fp32.  Allowed (in, work) pairs: (F32, F32), (BF16, F16),
 *   (BF16, BF16), (F16, F16).  (BF16, F16) is the precise choice for bf16
 *   inputs: fp16 keeps three more mantissa bits than bf16 at the same
 *   matrix-core rate, provided every intermediate stays below 65504 in
 *   magnitude (projected values of order one are far inside that range).
 *   Beyond it an fp16 intermediate becomes inf and the output is not
 *   finite; the call still returns MHA_OK (the library does not scan its
 *   intermediates).  Choose work_dtype = MHA_BF16 where range matters.
 * - The library allocates nothing, keeps no state between calls, never
 *   synchronises, and enqueues its kernels on `stream` (a hipStream_t; NULL
 *   means the null stream).  The caller owns every buffer; the one exception
 *   is the static scratch array of attn_core_split_noalloc (see there).
 * - Every argument that the host can check is checked before anything is
 *   launched; on error nothing is launched and nothing is written.
 * - Pointers must be aligned to their element size; 16-byte alignment and
 *   row widths that are multiples of 16 bytes select the vectorised paths.
 *
 * Device-side preconditions (not checked: they would need a device read)
 * ----------------------------------------------------------------------
 * - 0 <= key_len[b] <= n_k.
 * - Every query row has at least one allowed key (the summary definition
 *   requires nonempty allowed sets).  A row with none gets NaN outputs
 *   (0/0), row_m = -inf and row_l = 0.
 */
#ifndef MHA_H
#define MHA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MHA_OK = 0,
  MHA_ERR_NULL = -1,        /* a required pointer is NULL                           */
  MHA_ERR_DIM = -2,         /* a dimension is <= 0, or an index would overflow       */
  MHA_ERR_DTYPE = -3,       /* unknown dtype, or an unsupported (in, work) pair      */
  MHA_ERR_MASK = -4,        /* bad mask flags, causal with n_q != n_k, missing data  */
  MHA_ERR_ALIGN = -5,       /* a pointer is not aligned to its element size          */
  MHA_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than the *_workspace_bytes() */
  MHA_ERR_UNSUPPORTED = -7, /* d_h or d_vh above the largest instantiated head width */
  MHA_ERR_LAUNCH = -8,      /* the HIP runtime reported an error at launch           */
  MHA_ERR_SCALE = -9,       /* scale is not a finite number                          */
  MHA_ERR_SCRATCH = -10     /* attn_core_split_noalloc: the request exceeds the
                               library's static scratch (MHA_STATIC_SCRATCH_BYTES)    */
} mha_status;

typedef enum { MHA_F32 = 0, MHA_BF16 = 1, MHA_F16 = 2 } mha_dtype;

/* Mask rules, OR-able; 0 means every key is allowed.  The allowed set of a
 * query row is the AND of every selected rule.  Page "From Attention to
 * Self-Attention" review, "Distinctions to Keep": a causal mask removes
 * later positions, a padding mask removes artificial key positions, and the
 * two may be combined.  Page "Multi-head attention and self-attention",
 * Definition: any chosen mask, one for every head (there is no head axis). */
#define MHA_MASK_CAUSAL 1u      /* key j allowed for query i only if j <= i (needs n_q == n_k) */
#define MHA_MASK_KEY_PADDING 2u /* key j allowed only if j < key_len[b]                      */
#define MHA_MASK_BOOL 4u        /* key j allowed only if allowed[b][i][j] != 0               */
/* Additive score bias: review page "Multi-Head Attention", "The Complete
 * Multi-Head Operation", softmax(Q K^T / sqrt(d_k) + M).  M is added to the
 * scaled scores c q_i.k_j (it is not multiplied by c), one M for every head
 * (page "Multi-head attention and self-attention", Definition: one chosen
 * mask for every head).  Entries of -inf forbid the key
 * (as a rule above would); +inf and NaN entries are not allowed (not
 * checked: a device read).  A row whose allowed set ends up empty behaves
 * as described under the device-side preconditions above. */
#define MHA_MASK_ADDITIVE 8u    /* score_ij += add[b][i][j] (fp32)                          */

typedef struct mha_mask {
  uint32_t flags;               /* OR of MHA_MASK_* (unknown bits: MHA_ERR_MASK)            */
  const int32_t* key_len;       /* [B] valid keys per batch item (KEY_PADDING), device      */
  const uint8_t* allowed;       /* [Bm][n_q][n_k], 1 = allowed (BOOL), device               */
  int64_t allowed_batch_stride; /* elements between items; 0 = one mask for the batch       */
  const float* add;             /* [Ba][n_q][n_k] fp32 (ADDITIVE), device, 4-byte aligned   */
  int64_t add_batch_stride;     /* elements between items; 0 = one bias for the batch       */
} mha_mask;
/* Speed (not correctness) of the BOOL and ADDITIVE rules depends on layout:
 * with n_k and the batch strides multiples of 4 (and `add` 16-byte
 * aligned) the attention forward reads four keys' entries per load; a BOOL
 * mask alone with n_k and its batch stride multiples of 16, `allowed`
 * 16-byte aligned and n_q * n_k below 2^31 is moved into on-chip memory
 * with the key/value tiles (fastest).  Other layouts are read entry by
 * entry.  The causal and key-padding rules cost almost nothing: prefer them
 * to an equivalent BOOL mask. */

/* Projection biases (review page "Multi-Head Attention", "Parameter and
 * Work Conventions" and "Audit Order": the bias convention is stated, not
 * assumed).  Each pointer may be NULL (no bias for that product); a bias is
 * added to every row of its product in fp32, before the product is rounded:
 * Q W_Q + b_Q, K W_K + b_K, V W_V + b_V, Z W_O + b_O.  Element type
 * in_dtype, device memory, head r's part of b_Q / b_K / b_V in entries
 * r*d .. r*d+d-1 (the combined layout of the weights). */
typedef struct mha_bias {
  const void* b_Q;  /* [h*d_h]  */
  const void* b_K;  /* [h*d_h]  */
  const void* b_V;  /* [h*d_vh] */
  const void* b_O;  /* [d_o]    */
} mha_bias;

/* Dimensions use the general definition's names (page "Multi-head attention
 * and self-attention", Definition). */
typedef struct mha_dims {
  int32_t B;     /* batch items (independent; never mixed)            */
  int32_t h;     /* heads                                             */
  int32_t n_q;   /* query rows per item                               */
  int32_t n_k;   /* key / value rows per item                         */
  int32_t d_q;   /* query input width                                 */
  int32_t d_k;   /* key input width                                   */
  int32_t d_v;   /* value input width                                 */
  int32_t d_h;   /* per-head query/key width                          */
  int32_t d_vh;  /* per-head value width                              */
  int32_t d_o;   /* output width                                      */
  float scale;   /* score scale c; the usual choice is 1/sqrt(d_h)    */
  int32_t in_dtype;   /* mha_dtype of Q, K, V, weights (mha_forward) or
                          of Qh, Kh, Vh (attn_core)                    */
  int32_t out_dtype;  /* mha_dtype of Y (mha_forward) or Z (attn_core) */
  int32_t work_dtype; /* mha_forward intermediates (see above); ignored
                          by attn_core, whose weights use in_dtype      */
} mha_dims;

/* Bytes of scratch mha_forward needs for these dims: the projected heads
 * Qh [B,h,n_q,d_h], Kh [B,h,n_k,d_h], Vh [B,h,n_k,d_vh] and the
 * concatenation Z [B,n_q,h*d_vh], all in work_dtype, each 256-byte aligned.
 * Returns 0 if `d` is NULL or invalid. */
size_t mha_workspace_bytes(const mha_dims* d);

/* Full forward pass.  Page "Multi-head attention and self-attention",
 * Definition; review page "Multi-Head Attention", "The Complete Multi-Head
 * Operation".
 *   Q   [B, n_q, d_q]   K [B, n_k, d_k]   V [B, n_k, d_v]        (in_dtype)
 *   W_Q [d_q, h*d_h]    W_K [d_k, h*d_h]  W_V [d_v, h*d_vh]      (in_dtype)
 *   W_O [h*d_vh, d_o]                                            (in_dtype)
 *   bias  optional projection biases (NULL: none; see mha_bias)
 *   Y   [B, n_q, d_o]                                            (out_dtype, written)
 *   row_m, row_l  optional [B, h, n_q] fp32 (may be NULL): the final row
 *        maximum of the scaled scores (natural-log units) and the shifted
 *        normaliser sum_j exp(s_ij - row_m).
 *   workspace  device scratch of at least mha_workspace_bytes(d) bytes.
 * Q, K and V may alias (self-attention).  m may be NULL (no mask). */
mha_status mha_forward(const mha_dims* d, const mha_mask* m,
                       const void* Q, const void* K, const void* V,
                       const void* W_Q, const void* W_K, const void* W_V,
                       const void* W_O, const mha_bias* bias, void* Y,
                       float* row_m, float* row_l,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Attention on projected heads, written in the concatenated layout.
 * Page "Stable summary of an attention key block", Definition (summaries,
 * merge, final division); review page "Multi-Head Attention", shapes and
 * "Audit Order" (concatenate along the head-feature axis in head order).
 * Uses B, h, n_q, n_k, d_h, d_vh, scale, in_dtype, out_dtype of `d`.
 *   Qh [B, h, n_q, d_h]  Kh [B, h, n_k, d_h]  Vh [B, h, n_k, d_vh]   (in_dtype)
 *   Z  [B, n_q, h*d_vh]  head r in columns r*d_vh .. r*d_vh+d_vh-1   (out_dtype)
 *   row_m, row_l  optional, as for mha_forward. */
mha_status attn_core(const mha_dims* d, const mha_mask* m,
                     const void* Qh, const void* Kh, const void* Vh, void* Z,
                     float* row_m, float* row_l, void* stream);

/* Key-split form of attn_core, for few query rows against many keys
 * (decoding, short queries): the key axis is cut into partitions of whole
 * 64-key blocks, each partition of each row is summarised separately (m, l,
 * z) and the summaries are merged with the rule of page "Stable summary of
 * an attention key block", Definition (merge; the empty state, m = -inf,
 * l = 0, z = 0, is its identity), then z / l is written.  Same arguments,
 * masks, layouts and results as attn_core (up to fp32 rounding order), plus:
 *   splits     requested partitions, >= 0; 0 lets the library choose.  The
 *              count used is ceil(n_k / P), P = ceil(n_k / splits) rounded
 *              up to a multiple of 64 (at most 65536 partitions).
 *   workspace  device scratch of at least attn_split_workspace_bytes(d,
 *              splits) bytes, 256-byte aligned (hipMalloc's alignment):
 *              the partitions' fp32 summaries m, l [S, B, h, n_q] and
 *              z [S, B, h, n_q, d_vh].
 * Two launches on `stream`: the partitions, then the merge. */
size_t attn_split_workspace_bytes(const mha_dims* d, int32_t splits);
mha_status attn_core_split(const mha_dims* d, const mha_mask* m,
                           const void* Qh, const void* Kh, const void* Vh, void* Z,
                           float* row_m, float* row_l, int32_t splits,
                           void* workspace, size_t workspace_bytes, void* stream);

/* attn_core_split without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The partitions' summaries go to a
 * scratch array the library holds in each GPU's memory for the life of the
 * process (MHA_STATIC_SCRATCH_BYTES, 16 MiB); this call allocates nothing.
 * Same arguments, masks, layouts and results as attn_core_split (same
 * kernels, so bit for bit the same outputs), without workspace.  Errors as
 * there, plus MHA_ERR_SCRATCH when attn_split_workspace_bytes(d, splits)
 * exceeds MHA_STATIC_SCRATCH_BYTES (nothing is launched).  Every call on one
 * GPU shares that GPU's scratch: calls that overlap in time on one GPU (two
 * streams, or two host threads) race and may return wrong results; calls
 * ordered on one stream are safe.  Nothing in the scratch needs clearing:
 * each call writes every summary it reads. */
#define MHA_STATIC_SCRATCH_BYTES (16u << 20)
mha_status attn_core_split_noalloc(const mha_dims* d, const mha_mask* m,
                                   const void* Qh, const void* Kh, const void* Vh, void* Z,
                                   float* row_m, float* row_l, int32_t splits, void* stream);

/* Backward pass of attn_core: gradients of a scalar loss with respect to
 * Qh, Kh and Vh, given dZ, its gradient with respect to Z.  The pages define
 * the forward pass; the gradients follow from it by calculus (for one head,
 * A = softmax of S = c Qh Kh^T (+ M), Z = A Vh):
 *   dVh = A^T dZ,  dS = A o (dZ Vh^T - D),  D_i = sum_e dZ_ie Z_ie,
 *   dQh = c dS Kh, dKh = c dS^T Qh.
 * A is recomputed block by block from the forward's row statistics (page
 * "Stable summary of an attention key block", Definition: the weights are
 * e^(s - m) / l for the final (m, l) of each row); nothing of size n_q x n_k
 * is stored.  Same dims and mask as the forward call (an additive bias M is
 * applied; its gradient is attn_bias_backward's).
 *   in_dtype   BF16 or F16 (Qh, Kh, Vh: matrix-core kernels, operands
 *              rounded to that type, fp32 sums) or F32 (vector-ALU
 *              kernels, fp32 throughout).
 *   out_dtype  element type of Z, dZ and of the gradients written.
 *   Qh, Kh, Vh as for attn_core; Z [B, n_q, h*d_vh] the forward's output,
 *   dZ of the same shape; row_m, row_l [B, h, n_q] fp32 from the same
 *   forward call (required).
 *   dQh [B, h, n_q, d_h], dKh [B, h, n_k, d_h], dVh [B, h, n_k, d_vh]
 *   (written; keys no query may use get 0).
 *   workspace  device scratch of attn_backward_workspace_bytes(d) bytes,
 *   256-byte aligned (two fp32 values per row and head).
 * Three launches on `stream`: row terms, dKh and dVh, dQh.  The result is
 * deterministic (no atomics). */
size_t attn_backward_workspace_bytes(const mha_dims* d);
mha_status attn_core_backward(const mha_dims* d, const mha_mask* m,
                              const void* Qh, const void* Kh, const void* Vh,
                              const void* Z, const void* dZ,
                              const float* row_m, const float* row_l,
                              void* dQh, void* dKh, void* dVh,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Gradient of the same loss with respect to the additive score bias M of
 * attn_core (mask flag MHA_MASK_ADDITIVE required, else MHA_ERR_MASK).  M
 * enters every head's scores with coefficient 1 (page "Multi-Head Attention"
 * review, "The Complete Multi-Head Operation": softmax(Q K^T / sqrt(d_k) + M)
 * per head), so
 *   dM = sum over heads r of dS_r   (dS_r as in attn_core_backward),
 * summed over the batch items as well when one M serves them all
 * (add_batch_stride 0).  Arguments as for attn_core_backward (any in_dtype;
 * operands as the products of attn_core_backward see them: dZ rounded to
 * a 2-byte in_dtype), plus:
 *   dM  fp32 [B, n_q, n_k], or [1, n_q, n_k] for a shared M (written in
 *       full: entries that are forbidden, -inf in M, masked or past the
 *       keys of an item get 0), device memory, 4-byte aligned.
 *   workspace as for attn_core_backward (the row terms are formed again).
 * Two launches on `stream`: row terms, then one vector-ALU kernel that walks
 * the heads (and items) of each 64 x 64 tile of dM in order: deterministic,
 * no atomics, no scratch of size n_q x n_k per head. */
mha_status attn_bias_backward(const mha_dims* d, const mha_mask* m,
                              const void* Qh, const void* Kh, const void* Vh,
                              const void* Z, const void* dZ,
                              const float* row_m, const float* row_l, float* dM,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Gradient outputs for the projection biases of mha_backward: each pointer
 * may be NULL (not computed); element type out_dtype, device memory. */
typedef struct mha_bias_grad {
  void* db_Q;  /* [h*d_h]  */
  void* db_K;  /* [h*d_h]  */
  void* db_V;  /* [h*d_vh] */
  void* db_O;  /* [d_o]    */
} mha_bias_grad;

/* Scratch mha_backward needs for these dims, 256-byte aligned regions:
 * dZ, and the three heads' gradients in the concatenated layout (work_dtype),
 * the backward's row terms, the column-sum partials of the bias gradients,
 * the fp32 partial products of the K-split weight gradients, and (out_dtype
 * F32) dY rounded to work_dtype.  Returns 0 if `d` is NULL or invalid. */
size_t mha_backward_workspace_bytes(const mha_dims* d);

/* Backward pass of mha_forward: gradients of a scalar loss with respect to
 * the inputs, the weights and the biases, given dY, its gradient with
 * respect to Y.  The pages define the forward pass; the gradients are
 * calculus on it (page "Multi-head attention and self-attention",
 * Definition: Y = Concat(Z_1..Z_h) W^O with Z_r the attention of
 * (Q W_r^Q, K W_r^K, V W_r^V)):
 *   dZ = dY (W^O)^T, dW^O = Z^T dY, db_O = column sums of dY;
 *   per head, dQ_r, dK_r, dV_r from the core backward (attn_core_backward,
 *   the weights recomputed from the saved row statistics);
 *   dW^Q = Q^T dQ_cat, db_Q = column sums of dQ_cat, dQ = dQ_cat (W^Q)^T,
 *   likewise for K and V (dQ_cat: the heads' gradients side by side).
 * Arguments as for mha_forward (same dims and mask), plus:
 *   dY [B, n_q, d_o] (out_dtype); row_m, row_l [B, h, n_q] from the forward
 *   call (required); fwd_workspace: that call's workspace, still holding
 *   its projected heads and concatenation (fwd_workspace_bytes >=
 *   mha_workspace_bytes(d)).
 *   Outputs (out_dtype; any may be NULL and is then not computed):
 *   dQ [B, n_q, d_q], dK [B, n_k, d_k], dV [B, n_k, d_v] (written, not
 *   accumulated: for self-attention the gradient of X is dQ + dK + dV),
 *   dW_Q, dW_K, dW_V, dW_O (shapes of the weights), dbias (may be NULL).
 *   workspace: mha_backward_workspace_bytes(d) bytes, 256-byte aligned.
 * work_dtype BF16 or F16 (matrix-core core backward) or F32 (vector-ALU
 * core backward, fp32 operands).  All products accumulate in fp32;
 * operands are rounded to work_dtype.  Deterministic. */
mha_status mha_backward(const mha_dims* d, const mha_mask* m,
                        const void* Q, const void* K, const void* V,
                        const void* W_Q, const void* W_K, const void* W_V,
                        const void* W_O, const void* dY,
                        const float* row_m, const float* row_l,
                        const void* fwd_workspace, size_t fwd_workspace_bytes,
                        void* dQ, void* dK, void* dV,
                        void* dW_Q, void* dW_K, void* dW_V, void* dW_O,
                        const mha_bias_grad* dbias,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Static, human-readable name of a status code (host memory, never freed). */
const char* mha_status_string(int status);

/* Largest per-head widths the kernels are built for (d_h, d_vh). */
int32_t mha_max_head_dim(void);

#ifdef __cplusplus
}
#endif

#endif /* MHA_H */
