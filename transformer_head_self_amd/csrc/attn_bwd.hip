// Launches of the attention backward pass (matrix-core kernels for bf16 and
// fp16 heads; fp32 heads and the gradient of an additive score bias go to
// the vector-ALU kernels of attn_bwd_scalar.hpp).
#include "attn_bwd_scalar.hpp"

namespace mha {

template <typename T, int DH, int DV>
static hipError_t launch_bwd_fixed(const AttnBwdParams& p, hipStream_t stream) {
  const long long BH = (long long)p.B * p.h;
  const long long gkv = (long long)((p.n_k + 127) / 128) * BH;
  const long long gq = (long long)((p.n_q + 127) / 128) * BH;
  if (gkv > 2147483647LL || gq > 2147483647LL) return hipErrorInvalidValue;
  // Direct-to-LDS tiles for the dK/dV pass: 2-byte dZ of the heads' type,
  // exact widths of 64 or 128, 16-byte aligned rows, n_q a multiple of 4
  // (whole 16-byte chunks of the row terms), causal / key-padding masks only.
  constexpr bool dma_widths = (DH == 64 || DH == 128) && (DV == 64 || DV == 128);
  const bool dma = dma_widths && p.d_h == DH && p.d_vh == DV && p.z_dtype == p.elem_dtype &&
                   p.vec_q && p.vec_z && p.ldz % 8 == 0 && p.n_q % 4 == 0 &&
                   p.allowed == nullptr && p.add == nullptr;
  if (gkv > 0) {
    if constexpr (dma_widths) {
      if (dma) {
        hipLaunchKernelGGL((attn_bwd_kv_dma_kernel<T, DH, DV>), dim3((unsigned)gkv), dim3(256), 0,
                           stream, p);
      } else {
        hipLaunchKernelGGL((attn_bwd_kv_kernel<T, DH, DV>), dim3((unsigned)gkv), dim3(256), 0,
                           stream, p);
      }
    } else {
      hipLaunchKernelGGL((attn_bwd_kv_kernel<T, DH, DV>), dim3((unsigned)gkv), dim3(256), 0, stream,
                         p);
    }
  }
  // Direct-to-LDS key tiles for the dQ pass: K and V exactly 64 or 128
  // wide with 16-byte aligned rows, causal / key-padding masks only.
  const bool qdma = dma_widths && p.d_h == DH && p.d_vh == DV && p.vec_k && p.vec_v &&
                    p.allowed == nullptr && p.add == nullptr;
  if (gq > 0) {
    if constexpr (dma_widths) {
      if (qdma) {
        hipLaunchKernelGGL((attn_bwd_q_dma_kernel<T, DH, DV>), dim3((unsigned)gq), dim3(256), 0,
                           stream, p);
      } else {
        hipLaunchKernelGGL((attn_bwd_q_kernel<T, DH, DV>), dim3((unsigned)gq), dim3(256), 0,
                           stream, p);
      }
    } else {
      hipLaunchKernelGGL((attn_bwd_q_kernel<T, DH, DV>), dim3((unsigned)gq), dim3(256), 0, stream,
                         p);
    }
  }
  return hipGetLastError();
}

template <typename T, int DH>
static hipError_t launch_bwd_dv(const AttnBwdParams& p, hipStream_t stream) {
  if (p.d_vh <= 32) return launch_bwd_fixed<T, DH, 32>(p, stream);
  if (p.d_vh <= 64) return launch_bwd_fixed<T, DH, 64>(p, stream);
  if (p.d_vh <= 96) return launch_bwd_fixed<T, DH, 96>(p, stream);
  if (p.d_vh <= 128) return launch_bwd_fixed<T, DH, 128>(p, stream);
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_bwd_typed(const AttnBwdParams& p, hipStream_t stream) {
  if (p.d_h <= 32) return launch_bwd_dv<T, 32>(p, stream);
  if (p.d_h <= 64) return launch_bwd_dv<T, 64>(p, stream);
  if (p.d_h <= 128) return launch_bwd_dv<T, 128>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_row_terms(const AttnBwdParams& p, hipStream_t stream) {
  const size_t rows = (size_t)p.B * p.h * p.n_q;
  if (rows > 0) {
    const bool vec = p.z_dtype != kF32 && p.vec_z && p.ldz % 8 == 0 &&
                     (p.d_vh == 32 || p.d_vh == 64 || p.d_vh == 128);
    if (vec) {
      // 16-byte chunks, one per thread; 64 % (d_vh / 8) == 0, so one head's
      // chunks never straddle two waves
      const size_t blocks = ((size_t)p.B * p.n_q * p.ldz / 8 + 255) / 256;
      if (blocks > 2147483647ULL) return hipErrorInvalidValue;
      const dim3 grid((unsigned)blocks);
      const bool bf = p.z_dtype == kBF16;
      if (p.d_vh == 32) {
        if (bf) hipLaunchKernelGGL((attn_bwd_prep_vec_kernel<bf16, 4>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((attn_bwd_prep_vec_kernel<f16, 4>), grid, dim3(256), 0, stream, p);
      } else if (p.d_vh == 64) {
        if (bf) hipLaunchKernelGGL((attn_bwd_prep_vec_kernel<bf16, 8>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((attn_bwd_prep_vec_kernel<f16, 8>), grid, dim3(256), 0, stream, p);
      } else {
        if (bf) hipLaunchKernelGGL((attn_bwd_prep_vec_kernel<bf16, 16>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((attn_bwd_prep_vec_kernel<f16, 16>), grid, dim3(256), 0, stream, p);
      }
    } else {
      const size_t blocks = (rows + 3) / 4;   // four (row, head) waves per workgroup
      if (blocks > 2147483647ULL) return hipErrorInvalidValue;
      hipLaunchKernelGGL(attn_bwd_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    }
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_attention_backward(const AttnBwdParams& p, int elem_dtype, hipStream_t stream) {
  const hipError_t e = launch_bwd_row_terms(p, stream);
  if (e != hipSuccess) return e;
  switch (elem_dtype) {
    case kBF16: return launch_bwd_typed<bf16>(p, stream);
    case kF16: return launch_bwd_typed<f16>(p, stream);
    case kF32: return launch_attention_backward_scalar(p, stream);
    default: return hipErrorInvalidValue;
  }
}

// ---- vector-ALU kernels -----------------------------------------------
template <int DH, int DV>
static hipError_t launch_scalar_fixed(const AttnBwdParams& p, hipStream_t stream) {
  const long long BH = (long long)p.B * p.h;
  const long long gk = (long long)((p.n_k + 63) / 64) * BH;
  const long long gq = (long long)((p.n_q + 63) / 64) * BH;
  if (gk > 2147483647LL || gq > 2147483647LL) return hipErrorInvalidValue;
  if (gk > 0)
    hipLaunchKernelGGL((attn_bwd_kv_scalar_kernel<DH, DV>), dim3((unsigned)gk), dim3(256), 0,
                       stream, p);
  if (gq > 0)
    hipLaunchKernelGGL((attn_bwd_q_scalar_kernel<DH, DV>), dim3((unsigned)gq), dim3(256), 0,
                       stream, p);
  return hipGetLastError();
}

template <int DH, int DV>
static hipError_t launch_dm_fixed(const AttnBwdParams& p, float* dM, int shared,
                                  hipStream_t stream) {
  const long long Bo = shared ? 1 : p.B;
  const long long grid = (long long)((p.n_q + 63) / 64) * Bo * ((p.n_k + 63) / 64);
  if (grid > 2147483647LL) return hipErrorInvalidValue;
  if (grid > 0)
    hipLaunchKernelGGL((attn_bwd_dm_kernel<DH, DV>), dim3((unsigned)grid), dim3(256), 0, stream,
                       p, dM, shared);
  return hipGetLastError();
}

// Widths are rounded up to an instantiated tile (columns past d are zero).
template <template <int, int> class F, typename... A>
static hipError_t by_width(const AttnBwdParams& p, A... a) {
  auto dv = [&](auto dh) -> hipError_t {
    constexpr int DH = decltype(dh)::value;
    if (p.d_vh <= 32) return F<DH, 32>::run(p, a...);
    if (p.d_vh <= 64) return F<DH, 64>::run(p, a...);
    if (p.d_vh <= 96) return F<DH, 96>::run(p, a...);
    if (p.d_vh <= 128) return F<DH, 128>::run(p, a...);
    return hipErrorInvalidValue;
  };
  if (p.d_h <= 32) return dv(std::integral_constant<int, 32>{});
  if (p.d_h <= 64) return dv(std::integral_constant<int, 64>{});
  if (p.d_h <= 128) return dv(std::integral_constant<int, 128>{});
  return hipErrorInvalidValue;
}

template <int DH, int DV>
struct ScalarRun {
  static hipError_t run(const AttnBwdParams& p, hipStream_t s) {
    return launch_scalar_fixed<DH, DV>(p, s);
  }
};
template <int DH, int DV>
struct DmRun {
  static hipError_t run(const AttnBwdParams& p, float* dM, int shared, hipStream_t s) {
    return launch_dm_fixed<DH, DV>(p, dM, shared, s);
  }
};

hipError_t launch_attention_backward_scalar(const AttnBwdParams& p, hipStream_t stream) {
  return by_width<ScalarRun>(p, stream);
}

hipError_t launch_bias_backward(const AttnBwdParams& p, float* dM, int shared_bias,
                                hipStream_t stream) {
  if (p.add == nullptr) return hipErrorInvalidValue;
  return by_width<DmRun>(p, dM, shared_bias, stream);
}

}  // namespace mha
