// Projection GEMM for 2-byte elements on gfx950: C = A[M,K] * W[K,N].
//
// Same products and epilogues as gemm_kernel (page "Multi-head attention and
// self-attention", Definition: per-head projections and W^O; review page
// "Multi-Head Attention", "Separate and Combined Projections": the
// (B,T,h*d) -> (B,h,T,d) split folded into the store).  This variant is
// used when K is a multiple of 64, rows of A and W are 16-byte aligned and,
// for the head-major store, the head width is a multiple of 4.
//
// Design (ours): a 256 x 128 workgroup tile, four waves of 128 (rows of A)
// x 64 (columns of W); k advances 64 per LDS stage.  The product is computed
// transposed, C^T = W^T A^T, with 32x32x16 MFMAs, so each lane ends with four
// consecutive output columns of one row.  Both tiles are staged into LDS as
// plain 16-byte row copies; the W^T operand (one column of W, eight
// consecutive k per lane) is read with the transposing LDS load
// (ds_read_b64_tr_b16), which gathers four rows of a row-major tile into
// each lane.  Row pads keep both read patterns free of bank conflicts.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "gemm_store.hpp"
#include "internal.hpp"

namespace mha {

template <typename T>
struct Gemm2Cfg {
  static constexpr int BM = 256, BN = 128, BK = 64;
  static constexpr int NT = 256;
  static constexpr int VEC = 8;
  static constexpr int XROW = BK + 8;      // 144-byte rows: 16-byte reads of 32 rows spread
  static constexpr int WROW = BN + 32;     // 320-byte rows: 80 dwords, 16 mod 64
  static constexpr int X_PER_T = BM * BK / VEC / NT;   // 8
  static constexpr int W_PER_T = BK * BN / VEC / NT;   // 4
};

// T: element type of A, of the LDS tiles and of the MFMA operands (bf16/f16).
// TW: storage type of W (2 bytes); a W of the other kind is re-rounded to T
// (nearest even) as it is staged.
template <typename T, typename TW>
__global__ __launch_bounds__(256, 1) void gemm2_kernel(GemmBatch batch) {
  static_assert(sizeof(T) == 2 && sizeof(TW) == 2, "2-byte elements only");
  typedef Gemm2Cfg<T> C;
  typedef typename Elem<T>::vec vec;
  typedef typename Elem<T>::vec4 vec4;
  typedef typename Elem<TW>::vec wvec;
  constexpr int VEC = C::VEC;

  __shared__ __attribute__((aligned(16))) T Xs[C::BM * C::XROW];
  __shared__ __attribute__((aligned(16))) T Ws[C::BK * C::WROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;   // wave tile: rows wm*128.., columns wn*64..

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

  floatx16 acc[2][4];
  #pragma unroll
  for (int j = 0; j < 2; ++j)
    #pragma unroll
    for (int i = 0; i < 4; ++i)
      #pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.f;

  // Staging: thread chunk t covers row xr[t] (clamped into A, so rows past M
  // read valid memory; their results are never stored) and 8 columns of k;
  // W chunk t covers k row wr[t] and 8 columns (clamped below N the same way).
  // (element offsets fit in 32 bits: the host selects this kernel only then)
  int xsrc[C::X_PER_T], xdst[C::X_PER_T];
  #pragma unroll
  for (int t = 0; t < C::X_PER_T; ++t) {
    const int ci = tid + t * C::NT;
    const int row = ci / (C::BK / VEC), cc = ci % (C::BK / VEC);
    xsrc[t] = min(m0 + row, M - 1) * K + cc * VEC;
    xdst[t] = row * C::XROW + cc * VEC;
  }
  int wsrc[C::W_PER_T], wdst[C::W_PER_T];
  #pragma unroll
  for (int t = 0; t < C::W_PER_T; ++t) {
    const int ci = tid + t * C::NT;
    const int row = ci / (C::BN / VEC), cc = ci % (C::BN / VEC);
    wsrc[t] = row * N + min(n0 + cc * VEC, N - VEC);
    wdst[t] = row * C::WROW + cc * VEC;
  }
  vec xreg[C::X_PER_T];
  wvec wreg[C::W_PER_T];
  auto load_stage = [&](int k0) {
    #pragma unroll
    for (int t = 0; t < C::X_PER_T; ++t)
      xreg[t] = *reinterpret_cast<const vec*>(A + (unsigned)(xsrc[t] + k0));
    #pragma unroll
    for (int t = 0; t < C::W_PER_T; ++t)
      wreg[t] = *reinterpret_cast<const wvec*>(W + (unsigned)(wsrc[t] + k0 * N));
  };
  auto store_stage = [&]() {
    #pragma unroll
    for (int t = 0; t < C::X_PER_T; ++t) *reinterpret_cast<vec*>(&Xs[xdst[t]]) = xreg[t];
    #pragma unroll
    for (int t = 0; t < C::W_PER_T; ++t)
      *reinterpret_cast<vec*>(&Ws[wdst[t]]) = convert_chunk<T, TW>(wreg[t]);
  };

  // Per-lane read offsets.  X operand (B of the MFMA): row l32 of each
  // 32-row block, 8 consecutive k at 8*g.  W^T operand (A): the transposing
  // read, this lane addressing k row 8*g + (lane%16)/4 and 4 columns at
  // 16*((lane/16)%2) + 4*(lane%4) of each 32-column block.
  const int xoff = (wm * 128 + l32) * C::XROW + g * VEC;
  const int woff = (8 * g + ((lane & 15) >> 2)) * C::WROW + wn * 64 + 16 * ((lane >> 4) & 1) +
                   4 * (lane & 3);

  const int nstage = K / C::BK;
  load_stage(0);
  for (int s = 0; s < nstage; ++s) {
    __syncthreads();
    store_stage();
    __syncthreads();
    if (s + 1 < nstage) load_stage((s + 1) * C::BK);
    #pragma unroll
    for (int kc = 0; kc < C::BK / 16; ++kc) {
      vec wf[2], xf[4];
      #pragma unroll
      for (int j = 0; j < 2; ++j) {
        const T* wp = &Ws[woff + kc * 16 * C::WROW + j * 32];
        const vec4 lo = lds_read_tr4<T>(wp);
        const vec4 hi = lds_read_tr4<T>(wp + 4 * C::WROW);
        wf[j] = vec{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      #pragma unroll
      for (int i = 0; i < 4; ++i)
        xf[i] = *reinterpret_cast<const vec*>(&Xs[xoff + i * 32 * C::XROW + kc * 16]);
      #pragma unroll
      for (int j = 0; j < 2; ++j)
        #pragma unroll
        for (int i = 0; i < 4; ++i) mfma_chunk(acc[j][i], wf[j], xf[i]);
    }
  }

  store_wave_block_any(P, acc, m0 + wm * 128, n0 + wn * 64, g, l32);
}

}  // namespace mha
