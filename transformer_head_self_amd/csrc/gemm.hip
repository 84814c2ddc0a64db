// Launchers for the projection GEMM (fp32 and bf16 instantiations).
#include "gemm.hpp"

namespace mha {

// compute_dtype: element type of A and of the MFMA operands; w_dtype: storage
// type of W.  Supported pairs: (f32, f32), (bf16, bf16), (f16, f16), (f16, bf16).
hipError_t launch_gemm(const GemmBatch& in, int compute_dtype, int w_dtype, hipStream_t stream) {
  GemmBatch b = in;
  const int BM = 128, BN = 128;  // GemmCfg<T>::BM/BN for both element types
  int total = 0;
  for (int i = 0; i < b.count; ++i) {
    GemmProblem& p = b.p[i];
    p.tiles_m = (p.M + BM - 1) / BM;
    p.tiles_n = (p.N + BN - 1) / BN;
    p.tile_begin = total;
    total += p.tiles_m * p.tiles_n;
  }
  b.total_tiles = total;
  if (total == 0) return hipSuccess;
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
