// Launchers for the projection GEMM (fp32 and bf16 instantiations).
#include "gemm.hpp"

namespace mha {

hipError_t launch_gemm(const GemmBatch& in, int in_dtype, hipStream_t stream) {
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
  if (in_dtype == kBF16)
    hipLaunchKernelGGL(gemm_kernel<bf16>, dim3(total), dim3(256), 0, stream, b);
  else
    hipLaunchKernelGGL(gemm_kernel<float>, dim3(total), dim3(256), 0, stream, b);
  return hipGetLastError();
}

}  // namespace mha
