// Gradient GEMMs of the layer with direct global->LDS loads (gfx950),
// 2-byte operands: C[M, N] = A[M, K] * W[K, N] (fp32 accumulation) in the two
// layouts the backward of the projections needs:
//   AT = 0, WT = 1: A stored [M][K], W stored [N][K] (dZ = dY W_O^T,
//                   dX = dX_cat W^T: both factors contiguous along k);
//   AT = 1, WT = 0: A stored [K][M], W stored [K][N] (dW = X^T dX_cat,
//                   dW_O = Z^T dY: both factors contiguous along m / n).
// The products are calculus on page "Multi-head attention and
// self-attention", Definition (Y = Z W^O, Q_r = X W_r^Q, ...); see
// gemm_any.hpp for the general form these specialise.
//
// Design (ours), as gemm_dma_wide_kernel: 256 x 256 workgroup tile, eight
// waves of 128 x 64, C^T = W^T A^T with 32x32x16 MFMAs, 64-deep k stages
// (two of 64 KB in flight) moved by global_load_lds_dwordx4.  An operand
// contiguous along k is staged as 256 rows of 128 bytes and read with 16-byte
// row reads; one contiguous along m or n is staged as 64 k-rows of 512 bytes
// and read with the transposing LDS load.  The row permutations are the ones
// gemm_dma_wide_kernel uses for its two tiles (conflict-free for their read
// patterns).  Long-K products with few output tiles are split along K into
// fp32 partials that splitk_reduce_kernel sums in a fixed order.
#pragma once

#include "common.hpp"
#include "gemm.hpp"
#include "internal.hpp"
#include "lds_dma.hpp"

namespace mha {

struct GemmGradCfg {
  static constexpr int BM = 256, BN = 256, BK = 64, WAVES = 8;
  static constexpr int TILE = 32 * 1024;          // bytes per operand tile per stage
  static constexpr int INSTR = TILE / 1024 / WAVES;   // direct loads per wave per tile: 4
  static constexpr int A_AT = 0, W_AT = 2 * TILE;     // two stages of each operand
  static constexpr int LDS = 4 * TILE;                // 128 KB
};

// One operand tile of a stage.  KMAJ = false: 256 rows (m or n) of 64 k,
// 128-byte rows, chunk c of row r in slot c ^ ((r / 2) % 8).  KMAJ = true: 64
// k-rows of 256 elements, 512-byte rows, chunk c of row r in slot c ^ (4 (r % 4)).
template <bool KMAJ>
struct GradTile {
  // per-lane byte offset of direct load q (q < INSTR) of this wave, relative
  // to the operand's base at the stage's first k; r0: the tile's first row
  // (m or n) and R the number of rows; ld: row stride in elements
  __device__ __forceinline__ static unsigned load_off(int wave, int q, int lane, int r0, int R,
                                                      long long ld) {
    if constexpr (!KMAJ) {
      const int row = (wave * GemmGradCfg::INSTR + q) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((row >> 1) & 7);
      return (unsigned)(((long long)min(r0 + row, R - 1) * ld + c * 8) * 2);
    } else {
      const int row = (wave * GemmGradCfg::INSTR + q) * 2 + (lane >> 5);
      const int c = (lane & 31) ^ (4 * (row & 3));
      return (unsigned)(((long long)row * ld + min(r0 + c * 8, R - 8)) * 2);
    }
  }
  // bytes of one 64-deep k step in global memory
  __device__ __forceinline__ static long long k_step(long long ld) {
    return KMAJ ? 64 * ld * 2 : 128;
  }
};

template <typename T, typename TA, typename TW, bool AT, bool WT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_grad_kernel(GemmAny P) {
  static_assert(sizeof(T) == 2 && sizeof(TA) == 2 && sizeof(TW) == 2, "2-byte elements");
  static_assert(AT != WT, "layouts (A [M][K], W [N][K]) and (A [K][M], W [K][N])");
  typedef GemmGradCfg C;
  typedef typename Elem<T>::vec vec;
  typedef typename Elem<TA>::vec avec;
  typedef typename Elem<TA>::vec4 avec4;
  typedef typename Elem<TW>::vec wvec;
  typedef typename Elem<TW>::vec4 wvec4;
  typedef GradTile<AT> ATile;    // A contiguous along m: k-major tile
  typedef GradTile<!WT> WTile;   // W contiguous along n: k-major tile

  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  const unsigned lds_base = (unsigned)(size_t)(__attribute__((address_space(3))) char*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 2, wn = wave & 3;   // wave block: m rows wm*128.., n columns wn*64..

  // workgroup -> (K partition, output tile); partitions outer, so the
  // workgroups of one XCD share their K slices of A and W in its L2
  const int tiles_n = P.N / C::BN;
  const int tiles = (P.M / C::BM) * tiles_n;
  const int id = xcd_contiguous_tile(blockIdx.x, tiles * P.ksplit);
  const int ks = id / tiles;
  const int tile = id - ks * tiles;
  const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int kb = ks * P.kchunk;
  const int nstage = (min(P.K, kb + P.kchunk) - kb) / C::BK;

  const char* A = reinterpret_cast<const char*>(P.A) + (AT ? (long long)kb * P.lda * 2 : (long long)kb * 2);
  const char* W = reinterpret_cast<const char*>(P.W) + (WT ? (long long)kb * 2 : (long long)kb * P.ldw * 2);

  floatx16 acc[2][4];
  #pragma unroll
  for (int j = 0; j < 2; ++j)
    #pragma unroll
    for (int i = 0; i < 4; ++i)
      #pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.f;

  unsigned aoff[C::INSTR], woff[C::INSTR];
  #pragma unroll
  for (int q = 0; q < C::INSTR; ++q) {
    aoff[q] = ATile::load_off(wave, q, lane, m0, P.M, P.lda);
    woff[q] = WTile::load_off(wave, q, lane, n0, P.N, P.ldw);
  }
  const long long astep = ATile::k_step(P.lda), wstep = WTile::k_step(P.ldw);
  auto issue_stage = [&](int b, int s) {
    const char* As = A + s * astep;
    const char* Ws = W + s * wstep;
    const unsigned am = lds_base + C::A_AT + b * C::TILE + wave * C::INSTR * 1024;
    const unsigned wm0 = lds_base + C::W_AT + b * C::TILE + wave * C::INSTR * 1024;
    #pragma unroll
    for (int q = 0; q < C::INSTR; ++q) lds_dma16(As, aoff[q], am + q * 1024);
    #pragma unroll
    for (int q = 0; q < C::INSTR; ++q) lds_dma16(Ws, woff[q], wm0 + q * 1024);
  };

  // ---- per-lane LDS read offsets within a stage's tile (bytes) -------------
  // Row tile (128-byte rows): row r0 + 32 t + l32, chunk 2 kc + g; the
  // permutation depends on the row through l32 only.
  // k-major tile (512-byte rows), transposing read: k row 16 kc + 8 g +
  // (lane % 16) / 4 (+ 4 for the upper half) and columns c0 + 32 t +
  // 16 ((lane / 16) % 2) + 4 (lane % 4); one base per 32-column block t.
  auto row_off = [&](int r0, int kc) {
    const int r = r0 + l32;
    return r * 128 + (((2 * kc + g) ^ ((r >> 1) & 7)) * 16);
  };
  auto kmaj_off = [&](int c0) {
    const int kr = 8 * g + ((lane & 15) >> 2);
    const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    return kr * 512 + (((col >> 3) ^ (4 * (kr & 3))) * 16) + (col & 7) * 2;
  };
  // A: one base per 32-row block i (k-major) or per k-chunk kc (rows);
  // W: one base per 32-column block j (k-major) or per k-chunk kc (rows)
  int xo[4], wo[2], wro[4];
  if constexpr (AT) {
    #pragma unroll
    for (int i = 0; i < 4; ++i) xo[i] = kmaj_off(wm * 128 + 32 * i);
  } else {
    #pragma unroll
    for (int kc = 0; kc < 4; ++kc) xo[kc] = row_off(wm * 128, kc);
  }
  if constexpr (!WT) {
    #pragma unroll
    for (int j = 0; j < 2; ++j) wo[j] = kmaj_off(wn * 64 + 32 * j);
  } else {
    #pragma unroll
    for (int kc = 0; kc < 4; ++kc) wro[kc] = row_off(wn * 64, kc);
  }

  auto compute = [&](int b) {
    unsigned xs = lds_base + C::A_AT + b * C::TILE;
    unsigned ws = lds_base + C::W_AT + b * C::TILE;
    asm("" : "+s"(xs), "+s"(ws));
    #pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      vec wf[2], xf[4];
      #pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (!WT) {
          const unsigned p = ws + wo[j] + kc * 16 * 512;
          const wvec4 lo = lds_read_tr4_at<TW>(p);
          const wvec4 hi = lds_read_tr4_at<TW>(p + 4 * 512);
          wf[j] = convert_chunk<T, TW>(wvec{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        } else {
          wf[j] = convert_chunk<T, TW>(lds_load_at<wvec>(ws + wro[kc] + j * 32 * 128));
        }
      }
      #pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (AT) {
          const unsigned p = xs + xo[i] + kc * 16 * 512;
          const avec4 lo = lds_read_tr4_at<TA>(p);
          const avec4 hi = lds_read_tr4_at<TA>(p + 4 * 512);
          xf[i] = convert_chunk<T, TA>(avec{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        } else {
          xf[i] = convert_chunk<T, TA>(lds_load_at<avec>(xs + xo[kc] + i * 32 * 128));
        }
      }
      #pragma unroll
      for (int j = 0; j < 2; ++j)
        #pragma unroll
        for (int i = 0; i < 4; ++i) mfma_chunk(acc[j][i], wf[j], xf[i]);
    }
  };

  // one k stage in buffer b: wait until stage s has landed (nothing else is
  // outstanding); after the barrier no wave reads stage s-1, whose buffer
  // gets stage s+1
  if (nstage > 0) issue_stage(0, 0);
  for (int s = 0; s < nstage; ++s) {
    wait_vm_lds<0>();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    if (s + 1 < nstage) issue_stage((s + 1) & 1, s + 1);
    compute(s & 1);
  }

  // acc[j][i]: m = m0 + wm*128 + 32 i + l32, n = n0 + wn*64 + 32 j + 8 a + 4 g + (0..3)
  const int M = P.M, N = P.N;
  #pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + wm * 128 + 32 * i + l32;
    #pragma unroll
    for (int j = 0; j < 2; ++j)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int n = n0 + wn * 64 + 32 * j + 8 * a + 4 * g;
        if (P.ksplit > 1)
          store4(P.partial, kF32, ((size_t)ks * M + m) * N + n, true, 4, acc[j][i][4 * a],
                 acc[j][i][4 * a + 1], acc[j][i][4 * a + 2], acc[j][i][4 * a + 3]);
        else
          store4(P.C, P.c_dtype, (size_t)m * P.ldc + n, P.vec_c, N - n, acc[j][i][4 * a],
                 acc[j][i][4 * a + 1], acc[j][i][4 * a + 2], acc[j][i][4 * a + 3]);
      }
  }
}

}  // namespace mha
