// Epilogue shared by the 2-byte projection GEMMs: one wave's 128 x 64 block
// of C, held as acc[j][i] = rows m0w + 32 i + (lane % 32), columns
// n0w + 32 j + 8 a + 4 g + (0..3) in register 4a..4a+3 (g = lane / 32).
//
// kHeads: C is the head-major array (B, heads, ntok, dh) of page "Multi-head
// attention and self-attention", Definition (the per-head projections),
// stored as the split (B, T, h*d) -> (B, h, T, d) of review page
// "Multi-Head Attention", "Separate and Combined Projections"; row
// m = b*ntok + t, column n = r*dh + e.  The head width is a multiple of 4
// (host-checked), so four consecutive columns stay in one head.
// kRowMajor: C[m, n] row-major with N columns.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "fastdiv.hpp"
#include "internal.hpp"

namespace mha {

template <int DT, bool HEADS>
__device__ __forceinline__ void store_wave_block(const GemmProblem& P, const floatx16 (&acc)[2][4],
                                                 int m0w, int n0w, int g, int l32) {
  const int M = P.M, N = P.N;
  // column part of the destination offset, per (j, a)
  size_t coff[2][4];
  #pragma unroll
  for (int j = 0; j < 2; ++j)
    #pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int n = n0w + 32 * j + 8 * a + 4 * g;
      if constexpr (HEADS) {
        const int r = (int)fastdiv((uint32_t)n, P.dh_div);
        const int e = n - r * P.dh;
        coff[j][a] = (size_t)r * P.ntok * P.dh + e;
      } else {
        coff[j][a] = (size_t)n;
      }
    }
  const bool vec_ok = HEADS ? true : (P.vec_c && (N % 4) == 0);
  #pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0w + 32 * i + l32;
    if (m >= M) continue;
    size_t roff;
    if constexpr (HEADS) {
      const int bb = (int)fastdiv((uint32_t)m, P.ntok_div);
      const int t = m - bb * P.ntok;
      roff = ((size_t)bb * P.heads * P.ntok + t) * P.dh;
    } else {
      roff = (size_t)m * N;
    }
    #pragma unroll
    for (int j = 0; j < 2; ++j)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int n = n0w + 32 * j + 8 * a + 4 * g;
        if (n < N)
          store4(P.C, DT, roff + coff[j][a], vec_ok, N - n, acc[j][i][4 * a], acc[j][i][4 * a + 1],
                 acc[j][i][4 * a + 2], acc[j][i][4 * a + 3]);
      }
  }
}

// Dispatch on the problem's output layout and element type once, outside
// the unrolled stores, so the accumulators stay in registers.
__device__ __forceinline__ void store_wave_block_any(const GemmProblem& P,
                                                     const floatx16 (&acc)[2][4], int m0w,
                                                     int n0w, int g, int l32) {
  if (P.epilogue == kHeads) {
    if (P.out_dtype == kF32) store_wave_block<kF32, true>(P, acc, m0w, n0w, g, l32);
    else if (P.out_dtype == kBF16) store_wave_block<kBF16, true>(P, acc, m0w, n0w, g, l32);
    else store_wave_block<kF16, true>(P, acc, m0w, n0w, g, l32);
  } else {
    if (P.out_dtype == kF32) store_wave_block<kF32, false>(P, acc, m0w, n0w, g, l32);
    else if (P.out_dtype == kBF16) store_wave_block<kBF16, false>(P, acc, m0w, n0w, g, l32);
    else store_wave_block<kF16, false>(P, acc, m0w, n0w, g, l32);
  }
}

}  // namespace mha
