// Internal interfaces between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "fastdiv.hpp"

namespace mha {


// ---------------------------------------------------------------------------
// Projection GEMM: C = A[M,K] * W[K,N], both row-major, fp32 accumulation.
// Up to three independent problems per launch (the Q, K and V projections).
// Epilogue modes:
//   kHeads: column n -> head r = n / dh, e = n % dh; row m -> item b = m / ntok,
//           position t = m % ntok; stores out[((b*h + r)*ntok + t)*dh + e]
//           (the (B,T,h*d) -> (B,h,T,d) reshape/transpose folded into the store)
//   kRowMajor: out[m*N + n]
// ---------------------------------------------------------------------------
enum GemmEpilogue : int { kHeads = 0, kRowMajor = 1 };

struct GemmProblem {
  const void* A;     // [M, K]
  const void* W;     // [K, N]
  void* C;           // see epilogue
  int M, N, K;
  int epilogue;      // GemmEpilogue
  int out_dtype;     // DType of C
  int heads, dh, ntok;  // kHeads only
  int tiles_m, tiles_n, tile_begin;  // filled by the launcher
  int vec_a, vec_w;  // 16-byte vector loads allowed for A / W rows
  int vec_c;         // vector stores allowed for C (kRowMajor)
  const void* bias;  // optional [N], element type of W: C[m, n] += bias[n] before rounding
  FastDiv dh_div, ntok_div;  // filled by the launcher
};

struct GemmBatch {
  GemmProblem p[3];
  int count;
  int total_tiles;
};

hipError_t launch_gemm(const GemmBatch& batch, int compute_dtype, int w_dtype, hipStream_t stream);

// General product for the gradients: C[M, N] = A[M, K] * W[K, N] with either
// operand stored transposed (a_trans: A(m, k) = A[k*lda + m]; w_trans:
// W(k, n) = W[n*ldw + k]) and per-operand element types, computed in
// compute_dtype with fp32 accumulation; C row-major with row stride ldc.
struct GemmAny {
  const void* A;
  const void* W;
  void* C;
  int M, N, K;
  long long lda, ldw, ldc;
  int a_trans, w_trans;
  int a_dtype, w_dtype, c_dtype;
  int vec_a, vec_w, vec_c;   // vector loads / 4-element stores allowed (set by the launcher)
  int ksplit, kchunk;        // split-K (set by the launcher): ksplit partitions of kchunk
  float* partial;            // fp32 [ksplit, M, N] partial products when ksplit > 1
};
// `partial`: fp32 scratch of gemm_any_partial_floats(M, N, K) elements (may
// be NULL when that is 0).  Long-K products with few output tiles (the
// weight gradients) are split along K into partitions summed afterwards in a
// fixed order.
size_t gemm_any_partial_floats(int M, int N, int K);
hipError_t launch_gemm_any(GemmAny g, int compute_dtype, float* partial, hipStream_t stream);

// y = x rounded to y_dtype (bf16 or fp16, nearest even); n fp32 elements.
hipError_t launch_round_f32(const float* x, void* y, size_t n, int y_dtype, hipStream_t stream);

// out[n] = sum over m < M of X[m * ld + n] (n < N), in a fixed order;
// `part` is fp32 scratch of colsum_scratch_floats(M, N) elements.
size_t colsum_scratch_floats(int M, int N);
hipError_t launch_colsum(const void* X, int dtype, long long ld, int M, int N, void* out,
                         int out_dtype, float* part, hipStream_t stream);

// ---------------------------------------------------------------------------
// Fused attention: Z[b, i, r*d_vh + e] = sum_j softmax_j(c * q_i . k_j | mask) v_j[e]
// computed with running (m, l, z) summaries over key blocks.
// ---------------------------------------------------------------------------
struct AttnParams {
  const void* Q;     // [B, h, n_q, ldq]   (first d_h columns used)
  const void* K;     // [B, h, n_k, ldk]
  const void* V;     // [B, h, n_k, ldv]   (first d_vh columns used)
  void* Z;           // [B, n_q, ldz], head r at column r*d_vh
  float* row_m;      // optional [B, h, n_q]
  float* row_l;      // optional [B, h, n_q]
  const int32_t* key_len;   // optional [B]
  const uint8_t* allowed;   // optional [Bm, n_q, n_k]
  long long allowed_batch_stride;
  const float* add;         // optional additive score bias [Ba, n_q, n_k] (natural-log units)
  long long add_batch_stride;
  // allowed / add rows hold whole aligned groups of four keys (n_k and the
  // batch strides multiples of 4, allowed 4-byte and add 16-byte aligned):
  // the mask step reads four keys per load
  int mask_vec;
  // boolean rows also 16-byte aligned (n_k and the batch stride multiples
  // of 16) and n_q * n_k below 2^31: the direct-load kernel can move the
  // mask tile into LDS with the K/V tiles
  int mask_g16;
  int B, h, n_q, n_k, d_h, d_vh;
  int ldq, ldk, ldv, ldz;
  float scale_log2;  // c * log2(e)
  int causal;
  int out_dtype;
  int vec_q, vec_k, vec_v, vec_z;
  int num_q_tiles;   // filled by the launcher
  // Key-axis partitions (split launch only): partition sp covers keys
  // [sp * split_keys, (sp + 1) * split_keys) and writes its rows' partial
  // summaries instead of Z: part_m (maximum, base-2 units), part_l (the
  // normaliser at that shift) [splits, B, h, n_q] and part_z (the weighted
  // value sum at that shift) [splits, B, h, n_q, d_vh], all fp32; a row with
  // no allowed key in a partition gets the empty state (-inf, 0, 0).
  int splits;
  int split_keys;    // a multiple of 64
  float* part_m;
  float* part_l;
  float* part_z;
};

// elem_dtype: element type of Q, K, V (and of the softmax weights fed to
// the value product).
hipError_t launch_attention(const AttnParams& p, int elem_dtype, hipStream_t stream);

// The key-split form: the partial-summary launch (p.splits partitions of
// p.split_keys keys) followed by the merge launch that combines the
// partitions' summaries and writes Z (and row_m / row_l).
hipError_t launch_attention_split(const AttnParams& p, int elem_dtype, hipStream_t stream);

// ---------------------------------------------------------------------------
// Attention backward: gradients of a scalar loss with respect to Qh, Kh, Vh
// given dZ (its gradient with respect to the concatenated output) and the
// forward's row statistics (m, l).
// ---------------------------------------------------------------------------
struct AttnBwdParams {
  const void* Q;     // [B, h, n_q, d_h]   (element type T)
  const void* K;     // [B, h, n_k, d_h]
  const void* V;     // [B, h, n_k, d_vh]
  const void* Z;     // [B, n_q, ldz], head r at column r*d_vh   (z_dtype)
  const void* dZ;    // same layout and type as Z
  const float* row_m;  // [B, h, n_q] natural-log units
  const float* row_l;  // [B, h, n_q]
  void* dQ;          // [B, h, n_q, d_h]   (g_dtype)
  void* dK;          // [B, h, n_k, d_h]
  void* dV;          // [B, h, n_k, d_vh]
  float* lse2;       // workspace [B, h, n_q]: m log2(e) + log2(l), +inf for an empty row
  float* dsum;       // workspace [B, h, n_q]: sum_e dZ Z per row and head
  const int32_t* key_len;
  const uint8_t* allowed;
  long long allowed_batch_stride;
  const float* add;
  long long add_batch_stride;
  int B, h, n_q, n_k, d_h, d_vh;
  int ldz;
  float scale;       // c
  float scale_log2;  // c log2(e)
  int causal;
  int grad_concat;   // 1: dQ, dK, dV written in the concatenated layout
                     //    [B, n, h*d] (head r at columns r*d..), else head-major
  int elem_dtype;    // T: element type of Q, K, V and of the MFMA operands
  int z_dtype, g_dtype;
  int vec_q, vec_k, vec_v, vec_z;    // 16-byte loads allowed
  int vec_dq, vec_dk, vec_dv;        // 4-element vector stores allowed
};

// The launches of the backward pass on `stream`: the row terms (lse2,
// dsum), then dK/dV and dQ (matrix cores for 2-byte heads, the vector ALU
// for fp32 heads).
hipError_t launch_attention_backward(const AttnBwdParams& p, int elem_dtype, hipStream_t stream);

// The row terms alone (p.lse2, p.dsum from Z, dZ, row_m, row_l).
hipError_t launch_bwd_row_terms(const AttnBwdParams& p, hipStream_t stream);

// dK/dV and dQ on the vector ALU (any element type; row terms already formed).
hipError_t launch_attention_backward_scalar(const AttnBwdParams& p, hipStream_t stream);

// dM [Bo, n_q, n_k] (fp32; Bo = 1 when shared_bias, else B): the gradient
// with respect to the additive bias p.add, summed over heads (and items when
// shared); row terms already formed.
hipError_t launch_bias_backward(const AttnBwdParams& p, float* dM, int shared_bias,
                                hipStream_t stream);

// Largest head widths with an instantiated kernel.
constexpr int kMaxHeadDim = 128;

}  // namespace mha
