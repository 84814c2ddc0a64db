// Epilogue shared by the 2-byte projection GEMMs: one wave's (32 NI) x 64
// block of C (NI = 4 or 2), held as acc[j][i] = rows m0w + 32 i + (lane %
// 32), columns n0w + 32 j + 8 a + 4 g + (0..3) in register 4a..4a+3
// (g = lane / 32).
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

// Projection bias (the bias convention of review page "Multi-Head
// Attention", "Parameter and Work Conventions"): C[m, n] += bias[n], in fp32
// before the store rounds.  acc[j][i] holds columns n0w + 32 j + 8 a + 4 g +
// (0..3) in registers 4a..4a+3 for every i.  TW: the bias's element type
// (that of W).  Columns past N add nothing (they are never stored).
template <typename TW, int NI>
__device__ __forceinline__ void add_column_bias(const GemmProblem& P, floatx16 (&acc)[2][NI],
                                                int n0w, int g) {
  if (P.bias == nullptr) return;
  const TW* bias = reinterpret_cast<const TW*>(P.bias);
  #pragma unroll
  for (int j = 0; j < 2; ++j)
    #pragma unroll
    for (int a = 0; a < 4; ++a)
      #pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = n0w + 32 * j + 8 * a + 4 * g + e;
        const float bv = n < P.N ? (float)bias[n] : 0.f;
        #pragma unroll
        for (int i = 0; i < NI; ++i) acc[j][i][4 * a + e] += bv;
      }
}

template <int DT, bool HEADS, int NI>
__device__ __forceinline__ void store_wave_block(const GemmProblem& P, const floatx16 (&acc)[2][NI],
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
  for (int i = 0; i < NI; ++i) {
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

// The same stores staged through LDS so that every store instruction writes
// whole row segments: the wave writes its block into its own LDS region
// (rows padded by 16 bytes: the 8-byte writes of 32 rows and the 16-byte
// row reads both spread evenly over the banks), then reads back 16
// consecutive bytes per lane and stores them: 8 rows x 128 bytes per
// instruction for 2-byte outputs (one pass of 32 NI rows), 4 rows x 256
// bytes for fp32 (two passes of 16 NI rows).  With a head width of 64 a
// wave's block is one contiguous run of the head-major array.  `lds` is this
// wave's region of at least 32 NI x 144 bytes (18 KB for NI = 4), free for
// the wave's exclusive use; LDS
// operations of one wave complete in order, so no barrier is needed between
// the writes and the reads.  Conditions (checked by lds_store_ok): 2-byte
// head-major outputs need a head width that is a multiple of 8; row-major
// outputs need 16-byte aligned rows.
template <int DT, bool HEADS, int NI>
__device__ __forceinline__ void store_wave_block_lds(const GemmProblem& P,
                                                     const floatx16 (&acc)[2][NI], int m0w,
                                                     int n0w, int g, int l32, char* lds) {
  constexpr int ES = DT == kF32 ? 4 : 2;
  constexpr int ROWB = 64 * ES + 16;          // padded LDS row
  constexpr int ROWS = (DT == kF32 ? 16 : 32) * NI;  // rows per pass: at most 144 * 32 NI bytes
  constexpr int LPR = 64 * ES / 16;           // lanes per row in the read-back
  constexpr int RPI = 64 / LPR;               // rows per store instruction
  const int lane = g * 32 + l32;
  const int M = P.M, N = P.N;
  #pragma unroll
  for (int pass = 0; pass < 32 * NI / ROWS; ++pass) {
    // registers -> LDS: row (32 i + l32) - pass*ROWS, columns 32 j + 8 a + 4 g
    #pragma unroll
    for (int ii = 0; ii < ROWS / 32; ++ii) {
      const int i = pass * (ROWS / 32) + ii;
      #pragma unroll
      for (int j = 0; j < 2; ++j)
        #pragma unroll
        for (int a = 0; a < 4; ++a) {
          char* dst = lds + (ii * 32 + l32) * ROWB + (32 * j + 8 * a + 4 * g) * ES;
          const float v0 = acc[j][i][4 * a], v1 = acc[j][i][4 * a + 1];
          const float v2 = acc[j][i][4 * a + 2], v3 = acc[j][i][4 * a + 3];
          if constexpr (DT == kF32) {
            *reinterpret_cast<floatx4*>(dst) = floatx4{v0, v1, v2, v3};
          } else if constexpr (DT == kBF16) {
            *reinterpret_cast<bf16x4*>(dst) = Cvt<bf16>::four(v0, v1, v2, v3);
          } else {
            *reinterpret_cast<f16x4*>(dst) = Cvt<f16>::four(v0, v1, v2, v3);
          }
        }
    }
    // LDS -> global: lane covers row q / LPR of each group, 16 bytes at
    // column (q % LPR) * 16 / ES
    const int rq = lane / LPR, cq = (lane % LPR) * (16 / ES);
    const int n = n0w + cq;
    size_t coff = 0;
    if constexpr (HEADS) {
      const int r = (int)fastdiv((uint32_t)n, P.dh_div);
      coff = (size_t)r * P.ntok * P.dh + (n - r * P.dh);
    } else {
      coff = (size_t)n;
    }
    #pragma unroll
    for (int k = 0; k < ROWS / RPI; ++k) {
      const int row = k * RPI + rq;
      const int m = m0w + pass * ROWS + row;
      const uint4 v = *reinterpret_cast<const uint4*>(lds + row * ROWB + cq * ES);
      if (m < M && n < N) {
        size_t roff;
        if constexpr (HEADS) {
          const int bb = (int)fastdiv((uint32_t)m, P.ntok_div);
          const int t = m - bb * P.ntok;
          roff = ((size_t)bb * P.heads * P.ntok + t) * P.dh;
        } else {
          roff = (size_t)m * N;
        }
        *reinterpret_cast<uint4*>(reinterpret_cast<char*>(P.C) + (roff + coff) * ES) = v;
      }
    }
  }
}

__device__ __forceinline__ bool lds_store_ok(const GemmProblem& P) {
  const int es = P.out_dtype == kF32 ? 4 : 2;
  if (P.epilogue == kHeads) return es == 4 || (P.dh % 8) == 0;
  return P.vec_c && ((long long)P.N * es) % 16 == 0;
}

// Dispatch on the problem's output layout and element type once, outside
// the unrolled stores, so the accumulators stay in registers.
template <int NI>
__device__ __forceinline__ void store_wave_block_any(const GemmProblem& P,
                                                     const floatx16 (&acc)[2][NI], int m0w,
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

namespace mha {

// As store_wave_block_any, staged through `lds` when lds_store_ok(P).
template <int NI>
__device__ __forceinline__ void store_wave_block_any_lds(const GemmProblem& P,
                                                         const floatx16 (&acc)[2][NI], int m0w,
                                                         int n0w, int g, int l32, char* lds) {
  if (!lds_store_ok(P)) {
    store_wave_block_any(P, acc, m0w, n0w, g, l32);
    return;
  }
  if (P.epilogue == kHeads) {
    if (P.out_dtype == kF32) store_wave_block_lds<kF32, true>(P, acc, m0w, n0w, g, l32, lds);
    else if (P.out_dtype == kBF16) store_wave_block_lds<kBF16, true>(P, acc, m0w, n0w, g, l32, lds);
    else store_wave_block_lds<kF16, true>(P, acc, m0w, n0w, g, l32, lds);
  } else {
    if (P.out_dtype == kF32) store_wave_block_lds<kF32, false>(P, acc, m0w, n0w, g, l32, lds);
    else if (P.out_dtype == kBF16) store_wave_block_lds<kBF16, false>(P, acc, m0w, n0w, g, l32, lds);
    else store_wave_block_lds<kF16, false>(P, acc, m0w, n0w, g, l32, lds);
  }
}

}  // namespace mha
