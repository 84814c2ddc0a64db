#include <algorithm>

// Launchers for the projection GEMMs: the direct-to-LDS 2-byte kernel where
// its conditions hold, else the general 128x128 kernel (every element type).
#include "gemm.hpp"
#include "gemm_any.hpp"
#include "gemm_dma.hpp"
#include "gemm_dma_wide.hpp"
#include "gemm_grad.hpp"

namespace mha {

// compute_dtype: element type of A and of the MFMA operands; w_dtype: storage
// type of W.  Supported pairs: (f32, f32), (bf16, bf16), (f16, f16), (f16, bf16).
// The 256x128 direct-to-LDS kernel applies when every problem has K a multiple of
// 64, N a multiple of 8, 16-byte aligned rows, element offsets below 2^31
// (byte offsets below 2^32: the direct-to-LDS kernel's lane offsets)
// and (head-major store) a head width that is a multiple of 4.
static bool dma_gemm_applies(const GemmBatch& b, int compute_dtype, int w_dtype) {
  if (compute_dtype == kF32 || w_dtype == kF32) return false;
  for (int i = 0; i < b.count; ++i) {
    const GemmProblem& p = b.p[i];
    if (p.K % 64 != 0 || p.N % 8 != 0 || p.N < 8 || !p.vec_a || !p.vec_w) return false;
    if (p.epilogue == kHeads && p.dh % 4 != 0) return false;
    if ((long long)p.M * p.K >= (1LL << 31) || (long long)p.K * p.N >= (1LL << 31)) return false;
  }
  return true;
}

// The 256x256 tile with 64-deep stages (every A-tile row a whole 128-byte
// line) is used when every problem's N is a multiple of 256: measured 7 %
// faster on the Q/K/V projection of the 4x4096, d_model 1024 workload; with
// a ragged last column tile (N = 1152) its idle half cost more than it saved.
// With fewer than 128 such tiles (half the CUs or fewer busy) the 256x128
// tile runs twice as many workgroups: measured 37.0 -> 28.6 us on the output
// projection of the cross-attention workload (8192 x 768 x 1152, 96 tiles).
static bool wide_gemm_applies(const GemmBatch& b) {
  long long tiles = 0;
  for (int i = 0; i < b.count; ++i) {
    if (b.p[i].N % 256 != 0) return false;
    tiles += (long long)((b.p[i].M + 255) / 256) * (b.p[i].N / 256);
  }
  return tiles >= 128;
}


// With fewer 256 x 128 tiles than CUs, the 128 x 128 tile of the same kernel
// (four waves of 64 x 64) doubles the workgroups, and up to three share a CU
// (48 KB of LDS each) instead of one wave per SIMD working alone.
static constexpr long long kCUs = 256;   // MI355X
static bool half_gemm_applies(const GemmBatch& b) {
  long long tiles = 0;
  for (int i = 0; i < b.count; ++i)
    tiles += (long long)((b.p[i].M + 255) / 256) * ((b.p[i].N + 127) / 128);
  return tiles < kCUs;
}

hipError_t launch_gemm(const GemmBatch& in, int compute_dtype, int w_dtype, hipStream_t stream) {
  GemmBatch b = in;
  const bool big = dma_gemm_applies(b, compute_dtype, w_dtype);
  const bool wide = big && wide_gemm_applies(b);
  const bool half = big && !wide && half_gemm_applies(b);
  const int BM = big && !half ? 256 : 128, BN = wide ? 256 : 128;
  int total = 0;
  for (int i = 0; i < b.count; ++i) {
    GemmProblem& p = b.p[i];
    p.tiles_m = (p.M + BM - 1) / BM;
    p.tiles_n = (p.N + BN - 1) / BN;
    p.tile_begin = total;
    total += p.tiles_m * p.tiles_n;
    p.dh_div = make_fastdiv(p.dh > 0 ? (unsigned)p.dh : 1u);
    p.ntok_div = make_fastdiv(p.ntok > 0 ? (unsigned)p.ntok : 1u);
  }
  b.total_tiles = total;
  if (total == 0) return hipSuccess;
  if (wide) {
    if (compute_dtype == kBF16 && w_dtype == kBF16)
      hipLaunchKernelGGL((gemm_dma_wide_kernel<bf16, bf16>), dim3(total), dim3(512), 0, stream, b);
    else if (compute_dtype == kF16 && w_dtype == kF16)
      hipLaunchKernelGGL((gemm_dma_wide_kernel<f16, f16>), dim3(total), dim3(512), 0, stream, b);
    else if (compute_dtype == kF16 && w_dtype == kBF16)
      hipLaunchKernelGGL((gemm_dma_wide_kernel<f16, bf16>), dim3(total), dim3(512), 0, stream, b);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (big && half) {
    if (compute_dtype == kBF16 && w_dtype == kBF16)
      hipLaunchKernelGGL((gemm_dma_kernel<bf16, bf16, 2>), dim3(total), dim3(256), 0, stream, b);
    else if (compute_dtype == kF16 && w_dtype == kF16)
      hipLaunchKernelGGL((gemm_dma_kernel<f16, f16, 2>), dim3(total), dim3(256), 0, stream, b);
    else if (compute_dtype == kF16 && w_dtype == kBF16)
      hipLaunchKernelGGL((gemm_dma_kernel<f16, bf16, 2>), dim3(total), dim3(256), 0, stream, b);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (big) {
    if (compute_dtype == kBF16 && w_dtype == kBF16)
      hipLaunchKernelGGL((gemm_dma_kernel<bf16, bf16, 4>), dim3(total), dim3(256), 0, stream, b);
    else if (compute_dtype == kF16 && w_dtype == kF16)
      hipLaunchKernelGGL((gemm_dma_kernel<f16, f16, 4>), dim3(total), dim3(256), 0, stream, b);
    else if (compute_dtype == kF16 && w_dtype == kBF16)
      hipLaunchKernelGGL((gemm_dma_kernel<f16, bf16, 4>), dim3(total), dim3(256), 0, stream, b);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (compute_dtype == kBF16 && w_dtype == kBF16)
    hipLaunchKernelGGL((gemm_kernel<bf16, bf16>), dim3(total), dim3(256), 0, stream, b);
  else if (compute_dtype == kF16 && w_dtype == kF16)
    hipLaunchKernelGGL((gemm_kernel<f16, f16>), dim3(total), dim3(256), 0, stream, b);
  else if (compute_dtype == kF16 && w_dtype == kBF16)
    hipLaunchKernelGGL((gemm_kernel<f16, bf16>), dim3(total), dim3(256), 0, stream, b);
  else if (compute_dtype == kF32 && w_dtype == kF32)
    hipLaunchKernelGGL((gemm_kernel<float, float>), dim3(total), dim3(256), 0, stream, b);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

static bool aligned_to(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
static size_t elem_size(int dt) { return dt == kF32 ? 4 : 2; }

// Split-K partitions: only when the output has few tiles (fewer than 256
// workgroups) and K is long; about 512 workgroups, K chunks of at least 512.
static int gemm_any_splits(int M, int N, int K) {
  const long long tiles = (long long)((M + 127) / 128) * ((N + 127) / 128);
  if (tiles >= 256 || K < 1024) return 1;
  long long s = (512 + tiles - 1) / tiles;
  s = std::min<long long>(s, K / 512);
  return (int)std::max<long long>(s, 1);
}

// Direct-load gradient GEMM (gemm_grad_kernel): whole 256 x 256 tiles and
// 64-deep k stages.  Split-K when the output has fewer than 128 tiles and K
// is long: about 256 workgroups, K partitions of at least 1024 (multiples of
// 64).
static bool grad_dims_fit(int M, int N, int K) {
  return M > 0 && N > 0 && K > 0 && M % 256 == 0 && N % 256 == 0 && K % 64 == 0;
}
static int grad_splits(int M, int N, int K) {
  if (!grad_dims_fit(M, N, K)) return 1;
  const long long tiles = (long long)(M / 256) * (N / 256);
  if (tiles >= 128 || K < 2048) return 1;
  long long s = (256 + tiles - 1) / tiles;
  s = std::min<long long>(s, K / 1024);
  return (int)std::max<long long>(s, 1);
}

size_t gemm_any_partial_floats(int M, int N, int K) {
  const int s = std::max(gemm_any_splits(M, N, K), grad_splits(M, N, K));
  return s > 1 ? (size_t)s * M * N : 0;
}

// The direct-load gradient GEMM applies: 2-byte operands (both bf16 for a
// bf16 product), one of its two layouts, whole tiles, 16-byte aligned rows,
// byte offsets within a stage below 2^31.
static bool grad_gemm_applies(const GemmAny& g, int compute_dtype) {
  const bool two = g.a_dtype != kF32 && g.w_dtype != kF32;
  const bool types = compute_dtype == kF16
                         ? two
                         : (compute_dtype == kBF16 && g.a_dtype == kBF16 && g.w_dtype == kBF16);
  const bool layout = (g.a_trans == 0 && g.w_trans == 1) || (g.a_trans == 1 && g.w_trans == 0);
  if (!types || !layout || !grad_dims_fit(g.M, g.N, g.K) || !g.vec_a || !g.vec_w) return false;
  // row tiles: (rows - 1) * ld + 64 elements; k-major tiles: 64 * ld + rows
  const long long ra = g.a_trans ? 64LL * g.lda + g.M : (long long)g.M * g.lda;
  const long long rw = g.w_trans ? (long long)g.N * g.ldw : 64LL * g.ldw + g.N;
  return 2 * ra < (1LL << 31) && 2 * rw < (1LL << 31);
}

template <typename T, typename TA, typename TW>
static void launch_grad_typed(const GemmAny& g, dim3 grid, hipStream_t stream) {
  if (g.a_trans)
    hipLaunchKernelGGL((gemm_grad_kernel<T, TA, TW, true, false>), grid, dim3(512), 0, stream, g);
  else
    hipLaunchKernelGGL((gemm_grad_kernel<T, TA, TW, false, true>), grid, dim3(512), 0, stream, g);
}

static hipError_t launch_gemm_grad(GemmAny g, int compute_dtype, float* partial,
                                   hipStream_t stream) {
  g.ksplit = grad_splits(g.M, g.N, g.K);
  if (g.ksplit > 1 && partial == nullptr) return hipErrorInvalidValue;
  g.kchunk = g.ksplit > 1 ? ((g.K + g.ksplit - 1) / g.ksplit + 63) / 64 * 64 : g.K;
  g.ksplit = (g.K + g.kchunk - 1) / g.kchunk;
  g.partial = partial;
  const long long wgs = (long long)(g.M / 256) * (g.N / 256) * g.ksplit;
  if (wgs > 2147483647LL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs);
  if (compute_dtype == kBF16) {
    launch_grad_typed<bf16, bf16, bf16>(g, grid, stream);
  } else if (g.a_dtype == kBF16) {
    if (g.w_dtype == kBF16) launch_grad_typed<f16, bf16, bf16>(g, grid, stream);
    else launch_grad_typed<f16, bf16, f16>(g, grid, stream);
  } else {
    if (g.w_dtype == kBF16) launch_grad_typed<f16, f16, bf16>(g, grid, stream);
    else launch_grad_typed<f16, f16, f16>(g, grid, stream);
  }
  if (g.ksplit > 1) {
    const size_t n = (size_t)g.M * g.N;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, partial, g.ksplit, g.M, g.N, g.C, g.c_dtype, g.ldc);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_any(GemmAny g, int compute_dtype, float* partial, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const int vec = compute_dtype == kF32 ? 4 : 8;
  // chunks of `vec` elements along the contiguous dimension start at multiples
  // of `vec`; a full chunk is one or two aligned vector loads
  g.vec_a = aligned_to(g.A, 16) && g.lda % vec == 0;
  g.vec_w = aligned_to(g.W, 16) && g.ldw % vec == 0;
  g.vec_c = aligned_to(g.C, 4 * elem_size(g.c_dtype)) && g.ldc % 4 == 0;
  if (grad_gemm_applies(g, compute_dtype)) return launch_gemm_grad(g, compute_dtype, partial, stream);
  g.ksplit = gemm_any_splits(g.M, g.N, g.K);
  if (g.ksplit > 1 && partial == nullptr) return hipErrorInvalidValue;
  // K chunks are whole 32-element stages (vector loads stay aligned)
  g.kchunk = g.ksplit > 1 ? ((g.K + g.ksplit - 1) / g.ksplit + 31) / 32 * 32 : g.K;
  g.ksplit = (g.K + g.kchunk - 1) / g.kchunk;
  if (g.ksplit < 1) g.ksplit = 1;
  g.partial = partial;
  const long long tiles = (long long)((g.M + 127) / 128) * ((g.N + 127) / 128) * g.ksplit;
  if (tiles > 2147483647LL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tiles);
  if (compute_dtype == kBF16)
    hipLaunchKernelGGL(gemm_any_kernel<bf16>, grid, dim3(256), 0, stream, g);
  else if (compute_dtype == kF16)
    hipLaunchKernelGGL(gemm_any_kernel<f16>, grid, dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL(gemm_any_kernel<float>, grid, dim3(256), 0, stream, g);
  if (g.ksplit > 1) {
    const size_t n = (size_t)g.M * g.N;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, partial, g.ksplit, g.M, g.N, g.C, g.c_dtype, g.ldc);
  }
  return hipGetLastError();
}

hipError_t launch_round_f32(const float* x, void* y, size_t n, int y_dtype, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 2047) / 2048;   // eight elements per thread
  if (blocks > 2147483647ULL) return hipErrorInvalidValue;
  const int vec = aligned_to(x, 16) && aligned_to(y, 16);
  if (y_dtype == kBF16)
    hipLaunchKernelGGL(round_f32_kernel<bf16>, dim3((unsigned)blocks), dim3(256), 0, stream, x,
                       reinterpret_cast<bf16*>(y), n, vec);
  else
    hipLaunchKernelGGL(round_f32_kernel<f16>, dim3((unsigned)blocks), dim3(256), 0, stream, x,
                       reinterpret_cast<f16*>(y), n, vec);
  return hipGetLastError();
}

size_t colsum_scratch_floats(int M, int N) {
  return (size_t)((M + 255) / 256) * (size_t)N;
}

hipError_t launch_colsum(const void* X, int dtype, long long ld, int M, int N, void* out,
                         int out_dtype, float* part, hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  const int R = (M + 255) / 256;
  if (R > 0) {
    hipLaunchKernelGGL(colsum_partial_kernel, dim3((N + 255) / 256, R), dim3(256), 0, stream, X,
                       dtype, ld, M, N, part);
  }
  hipLaunchKernelGGL(colsum_finish_kernel, dim3((N + 255) / 256), dim3(256), 0, stream, part, R,
                     N, out, out_dtype);
  return hipGetLastError();
}

}  // namespace mha
