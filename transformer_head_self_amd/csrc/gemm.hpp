// Projection GEMMs for gfx950: C = A[M,K] * W[K,N], fp32 accumulation on
// the matrix cores, with the output layout chosen by the epilogue.
//
// Page "Multi-head attention and self-attention", Definition: each head has
// its own projections Q W_i^Q, K W_i^K, V W_i^V and the concatenated heads
// are multiplied by W^O.  Review page "Multi-Head Attention", "Separate and
// Combined Projections": with the heads' weights side by side, one wide
// product followed by (B,T,h*d) -> (B,T,h,d) -> (B,h,T,d) gives every head;
// here that reshape/transpose is folded into the store indexing (kHeads).
//
// Mapping onto the matrix cores (our design): the product is computed
// transposed, C^T = W^T A^T, with 32x32 MFMAs.  W is k-major in memory, so
// its tile is transposed on the way into LDS; afterwards both operands are
// read as 16-byte k-contiguous fragments.  In the result each lane holds
// four consecutive output columns of one row, which become one vector store
// in either output layout.
#pragma once

#include "common.hpp"
#include "gemm_store.hpp"
#include "internal.hpp"

namespace mha {

template <typename T>
struct GemmCfg {
  static constexpr int VEC = Elem<T>::VEC;
  static constexpr int BM = 128, BN = 128;      // workgroup tile
  static constexpr int WM = 64, WN = 64;        // wave tile (2 x 2 waves)
  static constexpr int NT = 256;
  static constexpr int KCH = 2;                 // k-chunks per LDS stage
  static constexpr int BK = KCH * 2 * VEC;      // 32 (bf16) / 16 (fp32)
  static constexpr int XPAD = BK + VEC;         // LDS row strides (elements)
  static constexpr int WPAD = BK + VEC;
  static constexpr int X_CHUNKS = BM * BK / VEC;
  static constexpr int W_CHUNKS = BK * BN / VEC;
  static constexpr int X_PER_T = X_CHUNKS / NT;
  static constexpr int W_PER_T = W_CHUNKS / NT;
  static_assert(X_CHUNKS % NT == 0 && W_CHUNKS % NT == 0, "tile/thread mismatch");
};

// Workgroup id -> tile id such that each XCD (workgroups are dispatched
// round-robin over 8 XCDs) receives one contiguous range of tiles.
__device__ __forceinline__ int xcd_contiguous_tile(int id, int total) {
  const int full = total / 8, rem = total % 8;
  const int x = id % 8, j = id / 8;
  return (x < rem) ? x * (full + 1) + j : rem * (full + 1) + (x - rem) * full + j;
}

// T: element type of A, of the LDS tiles and of the MFMA operands.
// TW: storage type of W (same size as T); a 2-byte W of the other kind is
// re-rounded to T (nearest even) as it is staged into LDS.
template <typename T, typename TW>
__global__ __launch_bounds__(256) void gemm_kernel(GemmBatch batch) {
  static_assert(sizeof(T) == sizeof(TW), "W must have the element size of T");
  typedef GemmCfg<T> C;
  typedef typename Elem<T>::vec vec;
  typedef typename Elem<TW>::vec wvec;
  constexpr int VEC = C::VEC;

  __shared__ __attribute__((aligned(16))) T Xs[C::BM * C::XPAD];
  __shared__ __attribute__((aligned(16))) T Wt[C::BN * C::WPAD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- which problem and tile --------------------------------------------
  const int tile = xcd_contiguous_tile(blockIdx.x, batch.total_tiles);
  int pi = 0;
  #pragma unroll
  for (int q = 1; q < 3; ++q)
    if (q < batch.count && tile >= batch.p[q].tile_begin) pi = q;
  // constant indices: the selected problem stays in scalar registers
  const GemmProblem P = (pi == 0) ? batch.p[0] : (pi == 1) ? batch.p[1] : batch.p[2];
  const int t_local = tile - P.tile_begin;
  const int tm = t_local / P.tiles_n;
  const int tn = t_local - tm * P.tiles_n;
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int M = P.M, N = P.N, K = P.K;
  const T* A = reinterpret_cast<const T*>(P.A);
  const TW* W = reinterpret_cast<const TW*>(P.W);
  const bool va = P.vec_a, vw = P.vec_w;

  floatx16 acc[2][2];
  #pragma unroll
  for (int j = 0; j < 2; ++j)
    #pragma unroll
    for (int i = 0; i < 2; ++i)
      #pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.f;

  vec xreg[C::X_PER_T];
  wvec wreg[C::W_PER_T];

  auto load_stage = [&](int k0) {
    #pragma unroll
    for (int t = 0; t < C::X_PER_T; ++t) {
      const int ci = tid + t * C::NT;
      const int row = ci / (C::BK / VEC);
      const int cc = ci - row * (C::BK / VEC);
      const int m = m0 + row;
      xreg[t] = (m < M) ? load_chunk<T>(A + (size_t)m * K + k0, cc * VEC, K - k0, va)
                        : zero_vec<vec>();
    }
    #pragma unroll
    for (int t = 0; t < C::W_PER_T; ++t) {
      const int ci = tid + t * C::NT;
      const int nc = ci / C::BK;         // consecutive threads: consecutive k rows
      const int kr = ci - nc * C::BK;
      const int k = k0 + kr;
      wreg[t] = (k < K) ? load_chunk<TW>(W + (size_t)k * N + n0, nc * VEC, N - n0, vw)
                        : zero_vec<wvec>();
    }
  };
  auto store_stage = [&]() {
    #pragma unroll
    for (int t = 0; t < C::X_PER_T; ++t) {
      const int ci = tid + t * C::NT;
      const int row = ci / (C::BK / VEC);
      const int cc = ci - row * (C::BK / VEC);
      *reinterpret_cast<vec*>(&Xs[row * C::XPAD + cc * VEC]) = xreg[t];
    }
    #pragma unroll
    for (int t = 0; t < C::W_PER_T; ++t) {
      const int ci = tid + t * C::NT;
      const int nc = ci / C::BK;
      const int kr = ci - nc * C::BK;
      const vec wv = convert_chunk<T, TW>(wreg[t]);
      #pragma unroll
      for (int e = 0; e < VEC; ++e) Wt[(nc * VEC + e) * C::WPAD + kr] = wv[e];
    }
  };

  const int nstage = (K + C::BK - 1) / C::BK;
  load_stage(0);
  for (int s = 0; s < nstage; ++s) {
    __syncthreads();
    store_stage();
    __syncthreads();
    if (s + 1 < nstage) load_stage((s + 1) * C::BK);
    #pragma unroll
    for (int kc = 0; kc < C::KCH; ++kc) {
      vec wf[2], xf[2];
      #pragma unroll
      for (int j = 0; j < 2; ++j)
        wf[j] = *reinterpret_cast<const vec*>(
            &Wt[(wn * C::WN + j * 32 + l32) * C::WPAD + kc * 2 * VEC + g * VEC]);
      #pragma unroll
      for (int i = 0; i < 2; ++i)
        xf[i] = *reinterpret_cast<const vec*>(
            &Xs[(wm * C::WM + i * 32 + l32) * C::XPAD + kc * 2 * VEC + g * VEC]);
      #pragma unroll
      for (int j = 0; j < 2; ++j)
        #pragma unroll
        for (int i = 0; i < 2; ++i) mfma_chunk(acc[j][i], wf[j], xf[i]);
    }
  }

  // ---- epilogue ------------------------------------------------------------
  add_column_bias<TW>(P, acc, n0 + wn * C::WN, g);
  #pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + wm * C::WM + i * 32 + l32;
    if (m >= M) continue;
    #pragma unroll
    for (int j = 0; j < 2; ++j) {
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int n = n0 + wn * C::WN + j * 32 + 8 * a + 4 * g;
        if (n >= N) continue;
        const float v[4] = {acc[j][i][4 * a], acc[j][i][4 * a + 1], acc[j][i][4 * a + 2],
                            acc[j][i][4 * a + 3]};
        if (P.epilogue == kRowMajor) {
          store4(P.C, P.out_dtype, (size_t)m * N + n, P.vec_c && (N % 4) == 0, N - n, v[0], v[1], v[2], v[3]);
        } else {
          const int bb = m / P.ntok, t = m - bb * P.ntok;
          if (P.dh % 4 == 0) {
            const int r = n / P.dh, e = n - r * P.dh;
            store4(P.C, P.out_dtype, (((size_t)bb * P.heads + r) * P.ntok + t) * P.dh + e, true,
                   N - n, v[0], v[1], v[2], v[3]);
          } else {
            #pragma unroll
            for (int q = 0; q < 4; ++q) {
              if (n + q >= N) break;
              const int r = (n + q) / P.dh, e = (n + q) - r * P.dh;
              store4(P.C, P.out_dtype, (((size_t)bb * P.heads + r) * P.ntok + t) * P.dh + e, false,
                     1, v[q], 0.f, 0.f, 0.f);
            }
          }
        }
      }
    }
  }
}

}  // namespace mha
