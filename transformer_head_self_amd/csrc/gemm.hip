// Launchers for the projection GEMMs: the direct-to-LDS 2-byte kernel where
// its conditions hold, else the general 128x128 kernel (every element type).
#include "gemm.hpp"
#include "gemm_dma.hpp"
#include "gemm_dma_wide.hpp"

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
static bool wide_gemm_applies(const GemmBatch& b) {
  for (int i = 0; i < b.count; ++i)
    if (b.p[i].N % 256 != 0) return false;
  return true;
}


hipError_t launch_gemm(const GemmBatch& in, int compute_dtype, int w_dtype, hipStream_t stream) {
  GemmBatch b = in;
  const bool big = dma_gemm_applies(b, compute_dtype, w_dtype);
  const bool wide = big && wide_gemm_applies(b);
  const int BM = big ? 256 : 128, BN = wide ? 256 : 128;
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
  if (big) {
    if (compute_dtype == kBF16 && w_dtype == kBF16)
      hipLaunchKernelGGL((gemm_dma_kernel<bf16, bf16>), dim3(total), dim3(256), 0, stream, b);
    else if (compute_dtype == kF16 && w_dtype == kF16)
      hipLaunchKernelGGL((gemm_dma_kernel<f16, f16>), dim3(total), dim3(256), 0, stream, b);
    else if (compute_dtype == kF16 && w_dtype == kBF16)
      hipLaunchKernelGGL((gemm_dma_kernel<f16, bf16>), dim3(total), dim3(256), 0, stream, b);
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

}  // namespace mha
