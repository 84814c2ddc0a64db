// Merge of key-partition summaries (the key-split form of the attention core).
//
// Page "Stable summary of an attention key block", Definition: two summaries
// (m1, l1, z1) and (m2, l2, z2) of disjoint key sets merge as m = max(m1, m2),
// l = l1 e^(m1 - m) + l2 e^(m2 - m), z = z1 e^(m1 - m) + z2 e^(m2 - m); the empty
// state (no allowed key: m = -inf, l = 0, z = 0) is the identity; the head
// output is z / l.  Here the partitions' summaries (base-2 units, written by
// attn_fwd_kernel's split form) are merged in partition order, one thread per
// output element, and z / l is written into the concatenation Z; a row with no
// allowed key anywhere gets 0 / 0 = NaN, as in the unsplit kernel.
#include "common.hpp"
#include "internal.hpp"

namespace mha {

__global__ __launch_bounds__(256) void split_merge_kernel(AttnParams p) {
  const size_t rows = (size_t)p.B * p.h * p.n_q;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * p.d_vh) return;
  const size_t rr = idx / p.d_vh;            // row = (b*h + r) * n_q + qi
  const int e = (int)(idx - rr * p.d_vh);
  float m = -INFINITY;
  for (int s = 0; s < p.splits; ++s) m = fmaxf(m, p.part_m[s * rows + rr]);
  float l = 0.f, z = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < p.splits; ++s) {
      const float ms = p.part_m[s * rows + rr];
      if (ms == -INFINITY) continue;          // empty partition: identity
      const float w = __builtin_amdgcn_exp2f(ms - m);
      l += p.part_l[s * rows + rr] * w;
      z += p.part_z[(s * rows + rr) * p.d_vh + e] * w;
    }
  }
  const int bh = (int)(rr / p.n_q);
  const int qi = (int)(rr - (size_t)bh * p.n_q);
  const int b = bh / p.h, r = bh - b * p.h;
  const size_t zi = ((size_t)b * p.n_q + qi) * p.ldz + (size_t)r * p.d_vh + e;
  const float v = z / l;
  if (p.out_dtype == kF32) reinterpret_cast<float*>(p.Z)[zi] = v;
  else if (p.out_dtype == kBF16) reinterpret_cast<bf16*>(p.Z)[zi] = (bf16)v;
  else reinterpret_cast<f16*>(p.Z)[zi] = (f16)v;
  if (e == 0) {
    if (p.row_m) p.row_m[rr] = (m == -INFINITY) ? -INFINITY : m * kLn2;
    if (p.row_l) p.row_l[rr] = l;
  }
}

hipError_t launch_split_merge(const AttnParams& p, hipStream_t stream) {
  const size_t n = (size_t)p.B * p.h * p.n_q * p.d_vh;
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  if (blocks > 2147483647ULL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(split_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mha
