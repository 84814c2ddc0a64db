// Three-stage software-pipelined fused attention forward for fp16 heads
// (gfx950).
//
// Computes what attn_fwd_kernel computes (page "Stable summary of an
// attention key block", Definition: per-row summaries merged block by block,
// z divided by l at the end; review page "Multi-Head Attention", "The
// Complete Multi-Head Operation": scaled scores, mask before the softmax,
// head result in its column block of the concatenation) for the common case:
// rows exactly d_h / d_vh wide and 16-byte aligned, causal and/or key-padding
// masks only, and no request for the final (m, l).
//
// Schedule (ours).  A wave owns 32 query rows, a workgroup four waves; key
// blocks of 64.  In iteration j a wave issues sixteen matrix instructions
// that do not depend on anything computed in the same iteration:
//   the value product of block j-1, O^T += V_{j-1}^T P_{j-1}^T (weights from
//   iteration j-1), and
//   the scores of block j+1, S_{j+1}^T = K_{j+1} Q^T - mu (the deferred
//   shift mu fed as the accumulator input),
// and between them the vector work of block j: its weights 2^(S_j - mu)
// (one exponential each), rounded to fp16, and their sum.  One matrix
// instruction of 32x32x16 keeps the matrix core busy for 32 cycles, during
// which the same wave can issue about four vector instructions, so each one
// is followed by four.  The order is pinned with scheduling barriers.
//
// Block order.  The summary merge does not depend on the order in which
// blocks are merged (page "Stable summary of an attention key block",
// Definition), so the workgroup walks its key blocks in the order: the
// blocks that some of its rows see only in part (causal diagonal, the last
// key-padding block), last block first, then every other block from 0 up.
// With 32-row waves and 64-key blocks a wave has at most one partly masked
// block, and it is the last block it uses at all; in this order it comes
// first, so it is also the wave's first block, whose exact maximum sets mu.
// Every later block needs no mask, and all waves end on the same block.
//
// LDS: K and V tiles travel in separate rings, K four stages deep and V
// five: in iteration j, K_{j+1} is read at the start for the scores, V_j
// during them for the value product of iteration j+1, and K_j stays
// available for a redo (see below).  Block j+3 is loaded in iteration j, so
// a tile has two iterations to arrive.
//
// Running state (deferred shift, as in attn_fwd_kernel's LAZY variant): o and
// l are kept at a reference shift mu set from the first block's exact
// maximum.  A lane's partial sum of a block's rounded weights bounds each of
// them; if it passes 2^8 (or overflows) the block is redone from its raw
// scores (formed again from K_j) with mu moved to the exact maximum, o and l
// are rescaled by the page's factor, and the next block's scores (already
// issued at the old shift) are moved too.
#pragma once

#include "attn.hpp"
#include "common.hpp"
#include "internal.hpp"
#include "lds_dma.hpp"

namespace mha {

// No instruction is scheduled across this point (the steady iteration's
// groups keep their source order).
#ifndef MHA_PIPE3_SCHED
#define MHA_PIPE3_SCHED 1
#endif
__device__ __forceinline__ void pipe_fence() {
#if MHA_PIPE3_SCHED
  __builtin_amdgcn_sched_barrier(0);
#endif
}
// Keeps a running sum's update in its group: without it the compiler sinks
// the additions below the later groups.
__device__ __forceinline__ void pin(float& x) {
#if MHA_PIPE3_SCHED
  asm volatile("" : "+v"(x));
#endif
}

template <typename T, int DH, int DV, int OCC = 2>
__global__ __launch_bounds__(256, OCC) void attn_fwd3_kernel(AttnParams p) {
  static_assert(__is_same(T, f16), "the deferred shift is used for fp16 heads");
  constexpr int WAVES = 4;
  constexpr int BN = 64;
  typedef AttnCfg<T, DH, DV, WAVES, BN> C;
  static_assert(C::KTILE == C::K_WIN * WAVES * 1024 && C::VTILE == C::V_WIN * WAVES * 1024,
                "every wave owns whole 1 KB load windows of both tiles");
  constexpr int NKB = C::NKB;    // 2 sub-blocks of 32 keys
  constexpr int KCH = C::KCH;    // 16-element k-chunks of a query row
  constexpr int NDV = C::NDV;    // 32-row blocks of V^T
  static_assert(NKB == 2, "64-key blocks");
  typedef typename Elem<T>::vec vec;
  typedef typename Elem<T>::vec4 vec4;
  typedef f16x2 pair;
  constexpr int VEC = C::VEC;
  constexpr int NSK = 4, NSV = 5;   // ring depths (tiles)

  __shared__ __attribute__((aligned(1024))) char smem[NSK * C::KTILE + NSV * C::VTILE];
  const unsigned lds_base = (unsigned)(size_t)(__attribute__((address_space(3))) char*)smem;
  const unsigned kring = lds_base;
  const unsigned vring = lds_base + NSK * C::KTILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;

  // Workgroup -> (query tile, batch*head) as in attn_fwd_kernel.
  const TileId tile = tile_of_workgroup(p, (int)blockIdx.x, false);
  const int qt = tile.qt, bh = tile.bh;
  const int b = bh / p.h;
  const int r = bh - b * p.h;
  const int q0 = qt * C::QT;
  const int qw = q0 + wave * 32;
  const int qi = qw + l32;

  int kvalid = p.n_k;
  if (p.key_len) kvalid = min(kvalid, p.key_len[b]);
  // Blocks [0, nblk) hold a key some row of the workgroup may use; blocks
  // [0, nfree_wg) need no mask for any of its rows.
  int kend = kvalid;
  if (p.causal) kend = min(kend, q0 + C::QT);
  const int nblk = kend > 0 ? (kend + BN - 1) / BN : 0;
  int nfree_wg = kvalid / BN;
  if (p.causal) nfree_wg = min(nfree_wg, (q0 + 1) / BN);
  nfree_wg = min(nfree_wg, nblk);
  const int ntail = nblk - nfree_wg;
  // Walk position j -> key block: the tail blocks last first, then the rest
  // from 0 up.
  auto block_at = [&](int j) { return j < ntail ? nblk - 1 - j : j - ntail; };
  // This wave uses blocks [0, nact), of which only block nact-1 may need a
  // mask (nfree: blocks no row of the wave masks); the walk reaches block
  // nact-1 at position jstart = nblk - nact, and every later position of
  // the walk is a block below nfree.
  int nact = 0, nfree = 0;
  if (qw < p.n_q) {
    const int klast = p.causal ? min(qw + 31, kvalid - 1) : kvalid - 1;
    nact = klast >= 0 ? min(nblk, klast / BN + 1) : 0;
    nfree = kvalid / BN;
    if (p.causal) nfree = min(nfree, (qw + 1) / BN);
  }
  const int jstart = nblk - nact;
  const bool first_masked = nfree < nact;

  const T* Qb = reinterpret_cast<const T*>(p.Q) + (size_t)bh * p.n_q * DH;
  const T* Kb = reinterpret_cast<const T*>(p.K) + (size_t)bh * p.n_k * DH;
  const T* Vb = reinterpret_cast<const T*>(p.V) + (size_t)bh * p.n_k * DV;

  // The query row scaled by c log2(e) (one rounding to T): scores arrive in
  // base-2 units.  Rows past n_q read the last row (never stored).
  vec qf[KCH];
  {
    const int qc = min(qi, p.n_q - 1);
    #pragma unroll
    for (int c = 0; c < KCH; ++c) {
      qf[c] = *reinterpret_cast<const vec*>(Qb + (size_t)qc * DH + c * 2 * VEC + g * VEC);
      #pragma unroll
      for (int e = 0; e < VEC; ++e) qf[c][e] = (T)((float)qf[c][e] * p.scale_log2);
    }
  }

  // ---- direct-to-LDS staging (row layouts and permutations as in
  // attn_fwd_kernel; K and V tiles in their own rings, slot = position) ------
  auto tile_row = [&](int win, int rb) { return (win * 1024 + 16 * lane) / rb; };
  auto k_chunk_of = [&](int win) {
    const int t = win * 1024 + 16 * lane, row = t / C::KRB;
    return ((t % C::KRB) / 16) ^ k_swizzle<C::KRB>(row);
  };
  auto v_chunk_of = [&](int win) {
    const int t = win * 1024 + 16 * lane, row = t / C::VRB;
    return ((t % C::VRB) / 16) ^ v_swizzle<C::VRB>(row);
  };
  unsigned koff[C::K_WIN], voff[C::V_WIN];
  #pragma unroll
  for (int q = 0; q < C::K_WIN; ++q) {
    const int win = wave * C::K_WIN + q;
    koff[q] = tile_row(win, C::KRB) * C::KRB + k_chunk_of(win) * 16;
  }
  #pragma unroll
  for (int q = 0; q < C::V_WIN; ++q) {
    const int win = wave * C::V_WIN + q;
    voff[q] = tile_row(win, C::VRB) * C::VRB + v_chunk_of(win) * 16;
  }
  // the tiles of walk position j into ring slots j % NSK and j % NSV
  auto issue_kv = [&](int j) {
    const int k0 = block_at(j) * BN;
    const unsigned ks = kring + (unsigned)((j % NSK) * C::KTILE);
    const unsigned vs = vring + (unsigned)((j % NSV) * C::VTILE);
    const char* kg = reinterpret_cast<const char*>(Kb) + (size_t)k0 * C::KRB;
    const char* vg = reinterpret_cast<const char*>(Vb) + (size_t)k0 * C::VRB;
    if (k0 + BN <= p.n_k) {
      #pragma unroll
      for (int q = 0; q < C::K_WIN; ++q) lds_dma16(kg, koff[q], ks + (wave * C::K_WIN + q) * 1024);
      #pragma unroll
      for (int q = 0; q < C::V_WIN; ++q) lds_dma16(vg, voff[q], vs + (wave * C::V_WIN + q) * 1024);
    } else {
      // a block running past n_k: its rows past n_k read the last key
      // (masked out, weight 0)
      const int last = p.n_k - 1 - k0;
      #pragma unroll
      for (int q = 0; q < C::K_WIN; ++q) {
        const int win = wave * C::K_WIN + q;
        lds_dma16(kg, min(tile_row(win, C::KRB), last) * C::KRB + k_chunk_of(win) * 16,
                  ks + win * 1024);
      }
      #pragma unroll
      for (int q = 0; q < C::V_WIN; ++q) {
        const int win = wave * C::V_WIN + q;
        lds_dma16(vg, min(tile_row(win, C::VRB), last) * C::VRB + v_chunk_of(win) * 16,
                  vs + win * 1024);
      }
    }
  };
  // Per-lane read offsets within a tile (bytes): K row kb*32 + l32, chunk
  // 2c + g; V the transposing read's rows 32 kb + 16 st + 8 h + 4 g +
  // (lane % 16) / 4, columns 32 d + scol (see attn_fwd_kernel).
  int kro[KCH], vro[NDV];
  #pragma unroll
  for (int c = 0; c < KCH; ++c)
    kro[c] = l32 * C::KRB + (((2 * c + g) ^ k_swizzle<C::KRB>(l32)) * 16);
  {
    const int vr = 4 * g + ((lane & 15) >> 2);
    const int scol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    #pragma unroll
    for (int d = 0; d < NDV; ++d) {
      const int ch = (d * 32 + scol) / 8;
      vro[d] = vr * C::VRB + ((ch ^ v_swizzle<C::VRB>(vr)) * 16) + (scol % 8) * 2;
    }
  }

  // ---- per-wave state ----------------------------------------------------------
  floatx16 o[NDV];
  #pragma unroll
  for (int d = 0; d < NDV; ++d)
    #pragma unroll
    for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
  float l_run = 0.f;   // this half-wave's part of the normaliser, at shift mu
  float mu = 0.f;
  floatx16 negmu;
  #pragma unroll
  for (int i = 0; i < 16; ++i) negmu[i] = 0.f;
  floatx16 sA[NKB], sB[NKB];   // scores of a block (two sets, roles alternate)
  vec pA[NKB][2], pB[NKB][2];  // weights of a block (two sets)
  vec vf[NKB][2][NDV];         // value fragments of the block whose value
                               // product comes next

  // K fragments of walk position j (A operands of the score product); the
  // tile's LDS address is made opaque so the per-read offsets become
  // instruction immediates
  auto read_k = [&](int j, vec (&kf)[NKB][KCH]) {
    unsigned st = kring + (unsigned)((j % NSK) * C::KTILE);
    asm("" : "+s"(st));
    #pragma unroll
    for (int c = 0; c < KCH; ++c) {
      unsigned a = st + (unsigned)kro[c];
      asm("" : "+v"(a));
      #pragma unroll
      for (int kb = 0; kb < NKB; ++kb) kf[kb][c] = lds_load_at<vec>(a + kb * 32 * C::KRB);
    }
  };
  // value fragments of walk position j (A operands of the value product),
  // piece u of 4 NDV (kb = u / (2 NDV), st2 = (u / NDV) % 2, d = u % NDV)
  auto vtile = [&](int j) {
    unsigned st = vring + (unsigned)((j % NSV) * C::VTILE);
    asm("" : "+s"(st));
    return st;
  };
  // per-lane base addresses of the value reads of one tile (one opaque
  // register per column block d; every other offset is an immediate)
  struct VBase { unsigned a[NDV]; };
  auto vbase = [&](int j) {
    const unsigned st = vtile(j);
    VBase vb;
    #pragma unroll
    for (int d = 0; d < NDV; ++d) {
      vb.a[d] = st + (unsigned)vro[d];
      asm("" : "+v"(vb.a[d]));
    }
    return vb;
  };
  auto read_v_piece = [&](const VBase& vb, int u) {
    const int kb = u / (2 * NDV), st2 = (u / NDV) % 2, d = u % NDV;
    const unsigned v0 = vb.a[d] + (kb * 32 + 16 * st2) * C::VRB;
    const vec4 lo = lds_read_tr4_at<T>(v0);
    const vec4 hi = lds_read_tr4_at<T>(v0 + 8 * C::VRB);
    vf[kb][st2][d] = vec{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  auto read_v = [&](int j) {
    const VBase vb = vbase(j);
    #pragma unroll
    for (int u = 0; u < 4 * NDV; ++u) read_v_piece(vb, u);
  };
  // weights of score pair t (scores 2t, 2t+1) of one sub-block: 2^(s - shift)
  // rounded to T, into slots 2(t%4), 2(t%4)+1 of chunk t/4; their sum into bsum
  const pair one2 = {(T)1.0f, (T)1.0f};
  auto exp_pair = [&](const floatx16& s, float shift, int t) {
    floatx2 e;
    e[0] = __builtin_amdgcn_exp2f(s[2 * t] - shift);
    e[1] = __builtin_amdgcn_exp2f(s[2 * t + 1] - shift);
    return e;
  };
  auto pack_pair = [&](floatx2 e, vec (&pc)[2], int t, float& bsum) {
    const pair w = __builtin_convertvector(e, pair);
    pc[t / 4][2 * (t % 4)] = w[0];
    pc[t / 4][2 * (t % 4) + 1] = w[1];
    bsum = __builtin_amdgcn_fdot2(w, one2, bsum, false);
  };
  auto weight_pair = [&](const floatx16& s, float shift, vec (&pc)[2], int t, float& bsum) {
    pack_pair(exp_pair(s, shift, t), pc, t, bsum);
  };
  // forbidden scores of key block blk -> -inf: causal and key padding allow
  // keys j <= lim (score slot (kb, i) of this lane is key
  // blk*64 + 32 kb + 8 (i / 4) + 4 g + i % 4)
  auto mask = [&](floatx16 (&s)[NKB], int blk) {
    const int lim = p.causal ? min(qi, kvalid - 1) : kvalid - 1;
    const int t = lim - blk * BN - 4 * g;
    #pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      #pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int off = kb * 32 + 8 * (i >> 2) + (i & 3);
        s[kb][i] = (off <= t) ? s[kb][i] : -INFINITY;
      }
  };
  auto block_max = [&](const floatx16 (&s)[NKB]) {
    float mx = -INFINITY;
    #pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      #pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    return half_max(mx);
  };
  auto rescale = [&](float a) {
    l_run *= a;
    #pragma unroll
    for (int d = 0; d < NDV; ++d)
      #pragma unroll
      for (int i = 0; i < 16; ++i) o[d][i] *= a;
  };
  auto value_mfma = [&](const vec (&pp)[NKB][2], int u) {
    const int kb = u / (2 * NDV), st2 = (u / NDV) % 2, d = u % NDV;
    mfma_chunk(o[d], vf[kb][st2][d], pp[kb][st2]);
  };
  // matrix step u of the scores of one block: accumulator -mu (or 0) + K Q^T
  auto score_mfma = [&](floatx16 (&sn)[NKB], const vec (&kf)[NKB][KCH], int u, bool at_mu) {
    const int kb = u / KCH, c = u % KCH;
    if (c == 0) {
      if (at_mu) {
        sn[kb] = negmu;
      } else {
        #pragma unroll
        for (int i = 0; i < 16; ++i) sn[kb][i] = 0.f;
      }
    }
    mfma_chunk(sn[kb], kf[kb][c], qf[c]);
  };
  // The weights of position j (an unmasked block) needed a redo (a weight
  // above 2^8, or an overflow): its raw scores are formed again from K_j
  // (still in its ring slot), mu moves up to their exact maximum, o and l
  // (they hold the blocks before j) are rescaled by the page's factor, the
  // weights are recomputed, and the next block's scores sn (issued at the
  // old shift, if `next`) are moved by the same amount.
  auto redo = [&](int j, floatx16 (&sn)[NKB], vec (&pc)[NKB][2], bool next, float& bsum) {
    compiler_fence();   // keep this rare path's reads out of the common path
    vec kf[NKB][KCH];
    read_k(j, kf);
    floatx16 t[NKB];
    #pragma unroll
    for (int u = 0; u < NKB * KCH; ++u) score_mfma(t, kf, u, false);
    const float mu_new = fmaxf(mu, block_max(t));
    const float dmu = mu_new - mu;
    rescale(__builtin_amdgcn_exp2f(-dmu));
    mu = mu_new;
    #pragma unroll
    for (int i = 0; i < 16; ++i) negmu[i] = -mu;
    bsum = 0.f;
    #pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      #pragma unroll
      for (int u = 0; u < 8; ++u) weight_pair(t[kb], mu, pc[kb], u, bsum);
    if (next) {
      #pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        #pragma unroll
        for (int i = 0; i < 16; ++i) sn[kb][i] -= dmu;
    }
  };

  // Iteration j of this wave's pipeline, jstart < j < nblk - 1: the value
  // product of position j-1 (weights pp, fragments vf read in iteration
  // j-1), the weights pc of position j (scores sc), the scores sn of
  // position j+1, all of unmasked blocks; position j's value fragments are
  // read for iteration j+1.
  auto steady = [&](int j, floatx16 (&sc)[NKB], floatx16 (&sn)[NKB], vec (&pp)[NKB][2],
                    vec (&pc)[NKB][2]) {
    // Sixteen groups, each fenced off so that the compiler keeps their
    // order: one matrix instruction (value product, then scores), the
    // exponentials of weight pair g, the rounding and row-sum step of pair
    // g-1 (one group later, so that no wait state is needed between an
    // exponential and its use), and in the second half two LDS reads.
    vec kf[NKB][KCH];
    read_k(j + 1, kf);
    float bsum = 0.f;
    floatx2 e = exp_pair(sc[0], 0.f, 0);
    value_mfma(pp, 0);
    pipe_fence();
    #pragma unroll
    for (int u = 1; u < 8; ++u) {
      value_mfma(pp, u);
      const floatx2 en = exp_pair(sc[0], 0.f, u);
      pack_pair(e, pc[0], u - 1, bsum);
      pin(bsum);
      e = en;
      pipe_fence();
    }
    const VBase vb = vbase(j);
    #pragma unroll
    for (int u = 0; u < 8; ++u) {
      score_mfma(sn, kf, u, true);
      read_v_piece(vb, u);
      const floatx2 en = exp_pair(sc[1], 0.f, u);
      if (u == 0)
        pack_pair(e, pc[0], 7, bsum);
      else
        pack_pair(e, pc[1], u - 1, bsum);
      pin(bsum);
      e = en;
      pipe_fence();
    }
    pack_pair(e, pc[1], 7, bsum);
    if (__any(!(bsum <= kLazyLimit))) redo(j, sn, pc, true, bsum);
    l_run += bsum;
  };
  constexpr int LOADS = C::K_WIN + C::V_WIN;   // per wave per position
  // Top of iteration j (every wave runs iterations -1 .. nblk, whatever its
  // rows use): position j+1 has landed once only position j+2's loads are
  // outstanding; after the barrier no wave reads K_{j-1} or V_{j-2} any
  // more, whose ring slots take position j+3.
  auto top = [&](int j) {
    if (j + 2 < nblk) wait_vm_lds<LOADS>();
    else wait_vm_lds<0>();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    if (j + 3 < nblk) issue_kv(j + 3);
  };
  auto copy_s = [&](floatx16 (&dst)[NKB], const floatx16 (&src)[NKB]) {
    #pragma unroll
    for (int kb = 0; kb < NKB; ++kb) dst[kb] = src[kb];
  };
  auto copy_p = [&](vec (&dst)[NKB][2], const vec (&src)[NKB][2]) {
    #pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      #pragma unroll
      for (int st = 0; st < 2; ++st) dst[kb][st] = src[kb][st];
  };

  // ---- the walk: positions 0 and 1 in flight, then iterations -1 .. nblk ------
  // Fill: iteration jstart-1 forms the raw scores of the wave's first
  // block, iteration jstart its mask, exact maximum (the first mu), weights
  // and the next block's scores; the steady iterations follow (two per trip,
  // the score and weight sets swapping roles, no branch inside); the drain
  // is iteration nblk-1 (value product, weights, no next scores) and
  // iteration nblk (the last value product).
  if (nblk > 0) issue_kv(0);
  if (nblk > 1) issue_kv(1);
  int j = -1;
  for (; j < jstart - 1; ++j) top(j);   // blocks none of this wave's rows use
  top(j);                                // j == jstart - 1
  if (nact > 0) {
    {
      vec kf[NKB][KCH];
      read_k(j + 1, kf);
      #pragma unroll
      for (int u = 0; u < NKB * KCH; ++u) score_mfma(sA, kf, u, false);
    }
    ++j;
    top(j);                              // j == jstart
    // the next block's raw scores go to the matrix cores first (they do not
    // depend on mu); the mask, the exact maximum and the weights of this
    // block run beside them, and mu is subtracted from those scores after
    const bool next = j + 1 < nblk;
    if (next) {
      vec kf[NKB][KCH];
      read_k(j + 1, kf);
      #pragma unroll
      for (int u = 0; u < NKB * KCH; ++u) score_mfma(sB, kf, u, false);
    }
    if (first_masked) mask(sA, block_at(j));
    // the exact maximum becomes mu; it is finite: this block holds each of
    // the wave's rows' last allowed key
    mu = block_max(sA);
    #pragma unroll
    for (int i = 0; i < 16; ++i) negmu[i] = -mu;
    {
      float bsum = 0.f;
      #pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        #pragma unroll
        for (int t = 0; t < 8; ++t) weight_pair(sA[kb], mu, pA[kb], t, bsum);
      l_run = bsum;
    }
    if (next) {
      #pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        #pragma unroll
        for (int i = 0; i < 16; ++i) sB[kb][i] -= mu;
    }
    read_v(j);
    ++j;
    // steady state: sc = sB (scores of position j), pp = pA (weights of j-1)
    for (; j + 2 < nblk; j += 2) {
      top(j);
      steady(j, sB, sA, pA, pB);
      top(j + 1);
      steady(j + 1, sA, sB, pB, pA);
    }
    if (j + 1 < nblk) {
      top(j);
      steady(j, sB, sA, pA, pB);
      ++j;
      copy_s(sB, sA);   // back to sc = sB, pp = pA (once per wave)
      copy_p(pA, pB);
    }
    if (j == nblk - 1) {
      top(j);
      // value product of position j-1 beside the weights of position j, in
      // the steady iteration's groups
      float bs0 = 0.f, bs1 = 0.f;
      #pragma unroll
      for (int u = 0; u < 8; ++u) {
        value_mfma(pA, u);
        weight_pair(sB[0], 0.f, pB[0], u, bs0);
        pin(bs0);
        pipe_fence();
      }
      #pragma unroll
      for (int t = 0; t < 8; ++t) weight_pair(sB[1], 0.f, pB[1], t, bs1);
      float bsum = bs0 + bs1;
      if (__any(!(bsum <= kLazyLimit))) redo(j, sA, pB, false, bsum);
      l_run += bsum;
      read_v(j);
      ++j;
      copy_p(pA, pB);
    }
    top(j);                              // j == nblk
    #pragma unroll
    for (int u = 0; u < 4 * NDV; ++u) value_mfma(pA, u);
  } else {
    top(j + 1);                          // j + 1 == nblk
  }

  // ---- finalise: z / l into the concatenation ---------------------------------
  const float l_tot = half_sum(l_run);
  const float inv = 1.0f / l_tot;
  if (qi < p.n_q) {
    const size_t zbase = ((size_t)b * p.n_q + qi) * p.ldz + (size_t)r * DV;
    #pragma unroll
    for (int d = 0; d < NDV; ++d)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int e0 = d * 32 + 8 * a + 4 * g;
        store4(p.Z, p.out_dtype, zbase + e0, p.vec_z, DV - e0, o[d][4 * a] * inv,
               o[d][4 * a + 1] * inv, o[d][4 * a + 2] * inv, o[d][4 * a + 3] * inv);
      }
  }
}

}  // namespace mha
