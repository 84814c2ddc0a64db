// Projection GEMM with direct global->LDS loads, 256x256 tiles and 64-deep
// k stages (gfx950), 2-byte elements.
//
// Same products, conditions and epilogues as gemm_dma_kernel (page
// "Multi-head attention and self-attention", Definition; review page
// "Multi-Head Attention", "Separate and Combined Projections").
//
// Why this shape (ours, measured): a direct load fetches whole 128-byte
// lines from L2, and rows of an A tile that are only 64 bytes deep (32 k)
// move at half the rate of full lines, the other half being evicted before
// the next stage could use it.  Here a stage is 64 k deep, so every A-tile
// row is one full line, and the 256x256 workgroup tile (eight waves of
// 128x64, one workgroup per CU) moves 60 % fewer line bytes per product than
// the 256x128 tile with 32-deep stages.  Two stages of 64 KB: the next stage
// loads while the current one is computed.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "gemm_store.hpp"
#include "internal.hpp"
#include "lds_dma.hpp"

namespace mha {

struct GemmWideCfg {
  static constexpr int BM = 256, BN = 256, BK = 64, NS = 2, WAVES = 8;
  static constexpr int NT = 64 * WAVES;
  static constexpr int XROWB = BK * 2;                 // 128-byte A-tile rows
  static constexpr int WROWB = BN * 2;                 // 512-byte W-tile rows
  static constexpr int XBYTES = BM * XROWB;            // 32 KB per stage
  static constexpr int WBYTES = BK * WROWB;            // 32 KB per stage
  static constexpr int X_INSTR = XBYTES / 1024 / WAVES;   // per wave per stage: 4
  static constexpr int W_INSTR = WBYTES / 1024 / WAVES;   // per wave per stage: 4
  static constexpr int KC = BK / 16;                   // MFMA k-chunks per stage
  static constexpr int X_AT = 0;
  static constexpr int W_AT = NS * XBYTES;
  static constexpr int STAGES = NS * (XBYTES + WBYTES);   // 128 KB
  static constexpr int EPILOGUE = WAVES * 128 * 144;      // staged stores, 18 KB per wave
  static constexpr int LDS = STAGES > EPILOGUE ? STAGES : EPILOGUE;   // 144 KB
};

// T: element type of A and of the MFMA operands; TW: storage type of W.
template <typename T, typename TW>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_dma_wide_kernel(GemmBatch batch) {
  static_assert(sizeof(T) == 2 && sizeof(TW) == 2, "2-byte elements only");
  typedef GemmWideCfg C;
  typedef typename Elem<T>::vec vec;
  typedef typename Elem<TW>::vec wvec;
  typedef typename Elem<TW>::vec4 wvec4;

  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int wm = wave >> 2, wn = wave & 3;   // wave block: rows wm*128.., columns wn*64..

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
  const char* A = reinterpret_cast<const char*>(P.A);
  const char* W = reinterpret_cast<const char*>(P.W);
  const unsigned lds_base = (unsigned)(size_t)(__attribute__((address_space(3))) char*)smem;

  floatx16 acc[2][4];
  #pragma unroll
  for (int j = 0; j < 2; ++j)
    #pragma unroll
    for (int i = 0; i < 4; ++i)
      #pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.f;

  // ---- direct loads: per-lane byte offsets for stage 0 ---------------------
  // A tile: rows of 128 bytes (64 k), 8 rows per wave instruction; chunk c of
  // row r (8 chunks of 8 k) is stored in slot c ^ ((r / 2) % 8), so 16
  // consecutive rows read at one chunk hit 16 distinct bank groups.  Rows past
  // M are clamped into A (read, never stored).
  // W tile: rows of 512 bytes (256 n), 2 rows per wave instruction; chunk c of
  // row r (32 chunks of 8 n) is stored in slot c ^ (4 * (r & 3)): the four
  // rows of one transposing-read phase land in distinct 64-byte bank quarters.
  // Columns past N are clamped to the last full chunk.
  unsigned xg[C::X_INSTR], wg[C::W_INSTR];
  #pragma unroll
  for (int q = 0; q < C::X_INSTR; ++q) {
    const int row = (wave * C::X_INSTR + q) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    xg[q] = ((unsigned)min(m0 + row, M - 1) * (unsigned)K + (unsigned)(c * 8)) * 2u;
  }
  #pragma unroll
  for (int q = 0; q < C::W_INSTR; ++q) {
    const int row = (wave * C::W_INSTR + q) * 2 + (lane >> 5);
    const int c = (lane & 31) ^ (4 * (row & 3));
    wg[q] = ((unsigned)row * (unsigned)N + (unsigned)min(n0 + c * 8, N - 8)) * 2u;
  }
  // stage s into buffer b (b == s % 2, a compile-time constant)
  auto issue_stage = [&](auto b, int s) {
    constexpr int B = decltype(b)::value;
    const char* As = A + (size_t)s * (C::BK * 2);
    const char* Ws = W + (size_t)s * C::BK * N * 2;
    const unsigned xm = lds_base + C::X_AT + B * C::XBYTES + wave * C::X_INSTR * 1024;
    const unsigned wm0 = lds_base + C::W_AT + B * C::WBYTES + wave * C::W_INSTR * 1024;
    #pragma unroll
    for (int q = 0; q < C::X_INSTR; ++q) lds_dma16(As, xg[q], xm + q * 1024);
    #pragma unroll
    for (int q = 0; q < C::W_INSTR; ++q) lds_dma16(Ws, wg[q], wm0 + q * 1024);
  };

  // ---- per-lane LDS read bases (bytes); the rest is immediate ------------
  // A operand (B of the MFMA): row r = wm*128 + 32 i + l32, chunk 2 kc + g;
  // 32 i does not change (r / 2) % 8, so i is an immediate.
  int xr[C::KC];
  #pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) {
    const int r = wm * 128 + l32;
    xr[kc] = r * C::XROWB + (((2 * kc + g) ^ ((r >> 1) & 7)) * 16);
  }
  // W^T operand (A of the MFMA), transposing read: this lane addresses k row
  // 16 kc + 8 g + (lane % 16) / 4 + 4 h and four columns at
  // wn*64 + 32 j + 16 ((lane / 16) % 2) + 4 (lane % 4); kc and h move the row by
  // multiples of 4 (same permutation: immediates); j selects one of two bases.
  int wr[2];
  #pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int kr = 8 * g + ((lane & 15) >> 2);
    const int col = wn * 64 + j * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int slot = (col >> 3) ^ (4 * (kr & 3));
    wr[j] = kr * C::WROWB + slot * 16 + (col & 7) * 2;
  }

  auto compute = [&](auto b) {
    constexpr int B = decltype(b)::value;
    const char* xs = smem + C::X_AT + B * C::XBYTES;
    const char* ws = smem + C::W_AT + B * C::WBYTES;
    #pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) {
      vec wf[2], xf[4];
      #pragma unroll
      for (int j = 0; j < 2; ++j) {
        const char* p = ws + wr[j] + kc * 16 * C::WROWB;
        const wvec4 lo = lds_read_tr4<TW>(reinterpret_cast<const TW*>(p));
        const wvec4 hi = lds_read_tr4<TW>(reinterpret_cast<const TW*>(p + 4 * C::WROWB));
        wf[j] = convert_chunk<T, TW>(wvec{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
      #pragma unroll
      for (int i = 0; i < 4; ++i)
        xf[i] = *reinterpret_cast<const vec*>(xs + xr[kc] + i * 32 * C::XROWB);
      #pragma unroll
      for (int j = 0; j < 2; ++j)
        #pragma unroll
        for (int i = 0; i < 4; ++i) mfma_chunk(acc[j][i], wf[j], xf[i]);
    }
  };

  typedef std::integral_constant<int, 0> B0;
  typedef std::integral_constant<int, 1> B1;
  const int nstage = K / C::BK;
  // One k stage in buffer b: wait until stage s has landed (nothing else is
  // outstanding); the same wait drains this wave's LDS reads of stage s-1, and
  // after the barrier no wave reads stage s-1, whose buffer gets stage s+1.
  auto step = [&](auto b, auto b1, int s) {
    wait_vm_lds<0>();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    if (s + 1 < nstage) issue_stage(b1, s + 1);
    compute(b);
  };
  issue_stage(B0(), 0);
  // pairs of stages, then an odd last one outside the loop: a conditional
  // second step inside the loop made the compiler copy the accumulators
  // between two register assignments on every iteration
  int s = 0;
  for (; s + 1 < nstage; s += 2) {
    step(B0(), B1(), s);
    step(B1(), B0(), s + 1);
  }
  if (s < nstage) step(B0(), B1(), s);

  // The epilogue's index arithmetic starts here (opaque copies of its inputs
  // keep the compiler from computing it before the loop).
  int m0w = m0 + wm * 128, n0w = n0 + wn * 64, lane_e = lane;
  asm volatile("" : "+s"(m0w), "+s"(n0w), "+v"(lane_e));
  add_column_bias<TW>(P, acc, n0w, lane_e >> 5);
  // every wave has finished reading the stage buffers before they are reused
  // for the staged stores (18 KB per wave)
  __syncthreads();
  store_wave_block_any_lds(P, acc, m0w, n0w, lane_e >> 5, lane_e & 31,
                           smem + wave * (128 * 144));
}

}  // namespace mha
