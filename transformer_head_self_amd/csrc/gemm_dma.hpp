// Projection GEMM with direct global->LDS loads (gfx950), 2-byte elements.
//
// Same products and epilogues as gemm_kernel (page "Multi-head
// attention and self-attention", Definition; review page "Multi-Head
// Attention", "Separate and Combined Projections").  Used for 2-byte A and W
// when K is a multiple of 64, N a multiple of 8, rows are 16-byte aligned
// and byte offsets into A and W fit in 32 bits.  A W stored in the other
// 2-byte type (bf16 weights with fp16 operands) is moved as stored and
// re-rounded (nearest even) after it is read from LDS.
//
// Design (ours): a 256 x 128 workgroup tile, four waves of 128 x 64, k
// stages of 32 (MI = 4); or, for grids that would leave CUs idle, a 128 x
// 128 tile of four waves of 64 x 64 (MI = 2: twice the workgroups, 48 KB of
// LDS, three workgroups per CU).  Tiles move from global memory into LDS with
// global_load_lds_dwordx4 (no staging registers): each wave instruction
// fills 1 KB of LDS, lane i writing bytes 16i..16i+15 of it from an address
// of its own choice (a fixed 32-bit lane offset from a scalar base that
// advances one stage at a time).  Three LDS stages are in flight; a stage is
// waited for with an explicit vector-memory count and a plain s_barrier (no
// memory fence, which would wait for the later stages too).  The stage loop
// is unrolled three times so every LDS address is a per-lane base plus an
// immediate.  Within a row the 16-byte chunks are XOR-permuted so that the
// 16-byte operand reads of A and the transposing reads of W hit distinct
// banks.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "gemm_store.hpp"
#include "internal.hpp"
#include "lds_dma.hpp"

namespace mha {

template <int MI>   // 32-row blocks of C per wave
struct GemmDmaCfg {
  static constexpr int BM = 64 * MI, BN = 128, BK = 32, NS = 3;
  static constexpr int NT = 256;
  static constexpr int XBYTES = BM * BK * 2;           // 16 KB per stage (MI = 4)
  static constexpr int WBYTES = BK * BN * 2;           // 8 KB per stage
  static constexpr int X_INSTR = XBYTES / 1024 / 4;    // per wave per stage: MI
  static constexpr int W_INSTR = WBYTES / 1024 / 4;    // per wave per stage: 2
  static constexpr int LOADS = X_INSTR + W_INSTR;      // vector-memory ops per wave per stage
  static constexpr int X_AT = 0;                       // X stages at 0, 16K, 32K
  static constexpr int W_AT = NS * XBYTES;             // W stages at 48K, 56K, 64K
  static constexpr int LDS = NS * (XBYTES + WBYTES);   // 72 KB (MI = 4): two workgroups per CU
  static constexpr int STAGE_OUT = 32 * MI * 144;      // staged stores per wave
  static_assert(LDS >= 4 * STAGE_OUT, "staging space for four waves");
};

// T: element type of A and of the MFMA operands; TW: storage type of W.
template <typename T, typename TW, int MI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_dma_kernel(GemmBatch batch) {
  static_assert(sizeof(T) == 2 && sizeof(TW) == 2, "2-byte elements only");
  static_assert(MI == 4 || MI == 2, "128 or 64 rows per wave");
  typedef GemmDmaCfg<MI> C;
  typedef typename Elem<T>::vec vec;
  typedef typename Elem<TW>::vec wvec;
  typedef typename Elem<TW>::vec4 wvec4;

  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;

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

  floatx16 acc[2][MI];
  #pragma unroll
  for (int j = 0; j < 2; ++j)
    #pragma unroll
    for (int i = 0; i < MI; ++i)
      #pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.f;

  // ---- direct loads: per-lane byte offsets for stage 0 ---------------------
  // A tile: rows of 64 bytes (32 k), 16 rows per wave instruction; chunk c of
  // row r (4 chunks of 8 k) is stored in slot c ^ ((r >> 2) & 3).  Rows past
  // M are clamped into A (read, never stored).
  // W tile: rows of 256 bytes (128 n), 4 rows per wave instruction; chunk c of
  // row r (16 chunks of 8 n) is stored in slot c ^ (4 * (r & 3)): the 32 lanes
  // of one transposing-read phase (4 rows, 2 x 16 columns) then cover all
  // banks.  Columns past N are clamped to the last full chunk.
  unsigned xg[C::X_INSTR], wg[C::W_INSTR];
  #pragma unroll
  for (int q = 0; q < C::X_INSTR; ++q) {
    const int row = (wave * C::X_INSTR + q) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    xg[q] = ((unsigned)min(m0 + row, M - 1) * (unsigned)K + (unsigned)(c * 8)) * 2u;
  }
  #pragma unroll
  for (int q = 0; q < C::W_INSTR; ++q) {
    const int row = (wave * C::W_INSTR + q) * 4 + (lane >> 4);
    const int c = (lane & 15) ^ (4 * (row & 3));
    wg[q] = ((unsigned)row * (unsigned)N + (unsigned)min(n0 + c * 8, N - 8)) * 2u;
  }
  // stage s into buffer b (b == s % 3, a compile-time constant)
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
  // A operand (B of the MFMA): row r = wm*32*MI + 32 i + l32, chunk 2 kc + g;
  // the slot permutation depends on r only through (r >> 2) & 3, which 32 i
  // does not change, so i is an immediate and kc selects one of two bases.
  int xr[2];
  #pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    const int r = wm * 32 * MI + l32;
    xr[kc] = r * 64 + (((2 * kc + g) ^ ((r >> 2) & 3)) * 16);
  }
  // W^T operand (A of the MFMA), transposing read: this lane addresses k row
  // 16 kc + 8 g + (lane % 16) / 4 + 4 h and four columns at
  // wn*64 + 32 j + 16 ((lane / 16) % 2) + 4 (lane % 4).  kc and h move the row
  // by multiples of 4 (same permutation: immediates); j selects one of two bases.
  int wr[2];
  #pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int kr = 8 * g + ((lane & 15) >> 2);
    const int col = wn * 64 + j * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int slot = (col >> 3) ^ (4 * (kr & 3));
    wr[j] = kr * 256 + slot * 16 + (col & 7) * 2;
  }

  auto compute = [&](auto b) {
    constexpr int B = decltype(b)::value;
    const char* xs = smem + C::X_AT + B * C::XBYTES;
    const char* ws = smem + C::W_AT + B * C::WBYTES;
    #pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      vec wf[2], xf[MI];
      #pragma unroll
      for (int j = 0; j < 2; ++j) {
        const char* p = ws + wr[j] + kc * 16 * 256;
        const wvec4 lo = lds_read_tr4<TW>(reinterpret_cast<const TW*>(p));
        const wvec4 hi = lds_read_tr4<TW>(reinterpret_cast<const TW*>(p + 4 * 256));
        wf[j] = convert_chunk<T, TW>(wvec{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
      #pragma unroll
      for (int i = 0; i < MI; ++i)
        xf[i] = *reinterpret_cast<const vec*>(xs + xr[kc] + i * 32 * 64);
      #pragma unroll
      for (int j = 0; j < 2; ++j)
        #pragma unroll
        for (int i = 0; i < MI; ++i) mfma_chunk(acc[j][i], wf[j], xf[i]);
    }
  };

  typedef std::integral_constant<int, 0> B0;
  typedef std::integral_constant<int, 1> B1;
  typedef std::integral_constant<int, 2> B2;
  const int nstage = K / C::BK;
  // One k stage in buffer b: wait until stage s has landed (only stage s+1's
  // loads may still be outstanding); the same wait drains this wave's LDS
  // reads of stage s-1, and after the barrier no wave reads stage s-1, whose
  // buffer b2 = (b + 2) % 3 is refilled with stage s+2.
  auto step = [&](auto b, auto b2, int s) {
    if (s + 1 < nstage) wait_vm_lds<C::LOADS>();
    else wait_vm_lds<0>();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    if (s + 2 < nstage) issue_stage(b2, s + 2);
    compute(b);
  };
  issue_stage(B0(), 0);
  if (1 < nstage) issue_stage(B1(), 1);
  // whole groups of three stages, then the rest outside the loop (no
  // conditional steps inside it: they made the compiler copy the
  // accumulators between register assignments on every iteration)
  int s = 0;
  for (; s + 2 < nstage; s += 3) {
    step(B0(), B2(), s);
    step(B1(), B0(), s + 1);
    step(B2(), B1(), s + 2);
  }
  if (s < nstage) step(B0(), B2(), s);
  if (s + 1 < nstage) step(B1(), B0(), s + 1);

  // The epilogue's index arithmetic starts here: opaque copies of its inputs
  // keep the compiler from computing it before the loop, where it would hold
  // registers across the whole k loop.
  int m0w = m0 + wm * 32 * MI, n0w = n0 + wn * 64, lane_e = lane;
  asm volatile("" : "+s"(m0w), "+s"(n0w), "+v"(lane_e));
  add_column_bias<TW>(P, acc, n0w, lane_e >> 5);
  // every wave has finished reading the stage buffers before they are reused
  // for the staged stores (18 KB per wave of the 72 KB at MI = 4)
  __syncthreads();
  store_wave_block_any_lds(P, acc, m0w, n0w, lane_e >> 5, lane_e & 31,
                           smem + wave * C::STAGE_OUT);
}

}  // namespace mha
