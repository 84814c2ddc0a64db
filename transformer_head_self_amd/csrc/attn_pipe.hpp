// Software-pipelined fused attention forward for 2-byte heads (gfx950).
//
// Computes what attn_fwd_kernel computes (page "Stable summary of an
// attention key block", Definition: per-row summaries merged block by block,
// z divided by l at the end; review page "Multi-Head Attention", "The
// Complete Multi-Head Operation": scaled scores, mask before the softmax,
// head result in its column block of the concatenation) for the common case:
// rows exactly d_h / d_vh wide and 16-byte aligned, causal and/or key-padding
// masks only, and no request for the final (m, l).
//
// Schedule (ours).  A wave owns 32 query rows, a workgroup four waves; K/V
// tiles of 64 keys move straight into LDS, three or four stages deep.  Within a
// wave the key blocks are software-pipelined: while the value product of
// block j runs on the matrix cores (O^T += V_j^T P_j^T), the wave computes
// the weights of block j+1 from its scores, which were issued just before
// (S_{j+1}^T = K_{j+1} Q^T - mu, the deferred shift mu fed as the MFMA's
// accumulator input).  The exponentials of one block thus overlap the matrix
// work of the neighbouring blocks instead of alternating with it.
//
// Running state (deferred shift, as in attn_fwd_kernel's LAZY variant): o and
// l are kept at a reference shift mu set from block 0's exact maximum.  A
// lane's partial sum of a block's rounded weights bounds each of them; if it
// passes 2^8 (or overflows) the block is redone from its raw scores with mu
// moved to the exact maximum, and o, l are rescaled by the page's factor.
#pragma once

#include "attn.hpp"
#include "common.hpp"
#include "internal.hpp"
#include "lds_dma.hpp"

namespace mha {

// NS: K/V stages in LDS (3 or 4); a block is loaded NS - 2 blocks ahead of
// its scores.  OCC: waves per SIMD the register allocation must allow.
// WAVES: waves per workgroup (4 or 8), 32 query rows each.
template <typename T, int DH, int DV, int NS = 4, int OCC = 2, int WAVES = 4>
__global__ __launch_bounds__(64 * WAVES, OCC) void attn_pipe_kernel(AttnParams p) {
  static_assert(sizeof(T) == 2, "2-byte heads");
  static_assert(NS == 3 || NS == 4, "three or four stages");
  static_assert(WAVES == 4 || WAVES == 8, "four or eight waves");
  constexpr int BN = 64;
  typedef AttnCfg<T, DH, DV, WAVES, BN> C;
  static_assert(C::KTILE == C::K_WIN * WAVES * 1024 && C::VTILE == C::V_WIN * WAVES * 1024,
                "every wave owns whole 1 KB load windows of both tiles");
  constexpr int NKB = C::NKB;   // 2 sub-blocks of 32 keys
  typedef typename Elem<T>::vec vec;
  typedef typename Elem<T>::vec4 vec4;
  constexpr int VEC = C::VEC;

  __shared__ __attribute__((aligned(1024))) char smem[NS * C::STAGE];
  const unsigned lds_base = (unsigned)(size_t)(__attribute__((address_space(3))) char*)smem;

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
  int kend = kvalid;
  if (p.causal) kend = min(kend, q0 + C::QT);
  const int nblk = kend > 0 ? (kend + BN - 1) / BN : 0;
  // This wave: blocks [0, nact) hold a key some of its rows may use; blocks
  // [0, nfree) need no mask for any of its rows.
  int nact = 0, nfree = 0;
  if (qw < p.n_q) {
    const int klast = p.causal ? min(qw + 31, kvalid - 1) : kvalid - 1;
    nact = min(nblk, klast / BN + 1);
    nfree = kvalid / BN;
    if (p.causal) nfree = min(nfree, (qw + 1) / BN);
  }

  const T* Qb = reinterpret_cast<const T*>(p.Q) + (size_t)bh * p.n_q * DH;
  const T* Kb = reinterpret_cast<const T*>(p.K) + (size_t)bh * p.n_k * DH;
  const T* Vb = reinterpret_cast<const T*>(p.V) + (size_t)bh * p.n_k * DV;

  // The query row scaled by c log2(e) (one rounding to T): scores arrive in
  // base-2 units.  Rows past n_q read the last row (never stored).
  vec qf[C::KCH];
  {
    const int qc = min(qi, p.n_q - 1);
    #pragma unroll
    for (int c = 0; c < C::KCH; ++c) {
      qf[c] = *reinterpret_cast<const vec*>(Qb + (size_t)qc * DH + c * 2 * VEC + g * VEC);
      #pragma unroll
      for (int e = 0; e < VEC; ++e) qf[c][e] = (T)((float)qf[c][e] * p.scale_log2);
    }
  }

  // ---- direct-to-LDS staging (same layout as attn_fwd_kernel's) -------------
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
  auto issue_kv = [&](int blk) {
    const int k0 = blk * BN;
    const unsigned st = lds_base + (unsigned)((blk % NS) * C::STAGE);
    const char* kg = reinterpret_cast<const char*>(Kb) + (size_t)k0 * C::KRB;
    const char* vg = reinterpret_cast<const char*>(Vb) + (size_t)k0 * C::VRB;
    if (k0 + BN <= p.n_k) {
      #pragma unroll
      for (int q = 0; q < C::K_WIN; ++q)
        lds_dma16(kg, koff[q], st + (wave * C::K_WIN + q) * 1024);
      #pragma unroll
      for (int q = 0; q < C::V_WIN; ++q)
        lds_dma16(vg, voff[q], st + C::KTILE + (wave * C::V_WIN + q) * 1024);
    } else {
      // last block: rows past n_k read the last key (masked out, weight 0)
      const int last = p.n_k - 1 - k0;
      #pragma unroll
      for (int q = 0; q < C::K_WIN; ++q) {
        const int win = wave * C::K_WIN + q;
        lds_dma16(kg, min(tile_row(win, C::KRB), last) * C::KRB + k_chunk_of(win) * 16,
                  st + win * 1024);
      }
      #pragma unroll
      for (int q = 0; q < C::V_WIN; ++q) {
        const int win = wave * C::V_WIN + q;
        lds_dma16(vg, min(tile_row(win, C::VRB), last) * C::VRB + v_chunk_of(win) * 16,
                  st + C::KTILE + win * 1024);
      }
    }
  };
  int kro[C::KCH], vro[C::NDV];
  #pragma unroll
  for (int c = 0; c < C::KCH; ++c)
    kro[c] = l32 * C::KRB + (((2 * c + g) ^ k_swizzle<C::KRB>(l32)) * 16);
  {
    const int vr = 4 * g + ((lane & 15) >> 2);
    const int scol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    #pragma unroll
    for (int d = 0; d < C::NDV; ++d) {
      const int ch = (d * 32 + scol) / 8;
      vro[d] = C::KTILE + vr * C::VRB + ((ch ^ v_swizzle<C::VRB>(vr)) * 16) + (scol % 8) * 2;
    }
  }

  // ---- per-wave state ----------------------------------------------------------
  floatx16 o[C::NDV];
  #pragma unroll
  for (int d = 0; d < C::NDV; ++d)
    #pragma unroll
    for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
  float l_run = 0.f;   // this half-wave's part of the normaliser, at shift mu
  float mu = 0.f;
  floatx16 negmu;
  #pragma unroll
  for (int i = 0; i < 16; ++i) negmu[i] = 0.f;
  vec pw[NKB][2];      // weights of the block whose value product is next
  floatx16 s[NKB];     // scores of the block after it

  // LDS byte address of a block's stage, opaque to the compiler: the reads
  // below add one per-lane offset to it and fold the rest into immediates
  // (left to itself the compiler kept a strength-reduced address per read).
  auto stage_ptr = [&](int blk) {
    unsigned a = lds_base + (unsigned)((blk % NS) * C::STAGE);
    asm("" : "+s"(a));
    return a;
  };
  // s = acc + K_blk Q^T  (acc = -mu or 0)
  auto scores = [&](unsigned st, bool at_mu) {
    unsigned kaddr[C::KCH];
    #pragma unroll
    for (int c = 0; c < C::KCH; ++c) {
      kaddr[c] = st + (unsigned)kro[c];
      asm("" : "+v"(kaddr[c]));
    }
    #pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (at_mu) {
        s[kb] = negmu;
      } else {
        #pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
      }
      #pragma unroll
      for (int c = 0; c < C::KCH; ++c) {
        const vec kf = lds_load_at<vec>(kaddr[c] + kb * 32 * C::KRB);
        mfma_chunk(s[kb], kf, qf[c]);
      }
    }
  };
  // forbidden scores -> -inf: causal and key padding allow keys j <= lim
  auto mask = [&](int blk) {
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
  auto block_max = [&]() {
    float mx = -INFINITY;
    #pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      #pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    return half_max(mx);
  };
  // weights of sub-block kb, rounded to T, summed into bsum
  auto weights = [&](int kb, float shift, float& bsum) {
    #pragma unroll
    for (int st = 0; st < 2; ++st) {
      floatx8 pf;
      #pragma unroll
      for (int t = 0; t < 8; ++t) pf[t] = __builtin_amdgcn_exp2f(s[kb][8 * st + t] - shift);
      pw[kb][st] = Cvt<T>::eight(pf);
      bsum = sum8(pw[kb][st], bsum);
    }
  };
  // o += V_blk^T P^T for the weights in pw (sub-block kb)
  auto value_product = [&](unsigned st, int kb) {
    unsigned vaddr[C::NDV];
    #pragma unroll
    for (int d = 0; d < C::NDV; ++d) {
      vaddr[d] = st + (unsigned)vro[d];
      asm("" : "+v"(vaddr[d]));
    }
    #pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      #pragma unroll
      for (int d = 0; d < C::NDV; ++d) {
        const unsigned v0 = vaddr[d] + (kb * 32 + 16 * h2) * C::VRB;
        const vec4 lo = lds_read_tr4_at<T>(v0);
        const vec4 hi = lds_read_tr4_at<T>(v0 + 8 * C::VRB);
        const vec va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        mfma_chunk(o[d], va, pw[kb][h2]);
      }
  };
  auto rescale = [&](float a) {
    l_run *= a;
    #pragma unroll
    for (int d = 0; d < C::NDV; ++d)
      #pragma unroll
      for (int i = 0; i < 16; ++i) o[d][i] *= a;
  };

  // ---- prologue: NS - 1 stages in flight, block 0's weights at its maximum -
  constexpr int LOADS = C::K_WIN + C::V_WIN;   // per wave per block
  if (nblk > 0) issue_kv(0);
  if (nblk > 1) issue_kv(1);
  if (NS == 4 && nblk > 2) issue_kv(2);
  if (NS == 4 && nblk > 2) wait_vm_lds<2 * LOADS>();
  else if (nblk > 1) wait_vm_lds<LOADS>();
  else wait_vm_lds<0>();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
  if (nact > 0) {
    scores(stage_ptr(0), false);
    if (nfree == 0) mask(0);
    const float mx = block_max();   // finite: key 0 is allowed for every row
    mu = mx;
    #pragma unroll
    for (int i = 0; i < 16; ++i) negmu[i] = -mu;
    float b0 = 0.f;
    weights(0, mu, b0);
    weights(1, mu, b0);
    l_run = b0;
  }

  // ---- main loop: block j's value product overlaps block j+1's weights -----
  for (int j = 0; j < nblk; ++j) {
    if (j + 1 < nblk) {
      // block j+1 has landed once only the loads of the blocks issued after
      // it (block j+2, with four stages) are outstanding; after the barrier
      // no wave reads block j-1, whose stage gets block j + NS - 1
      if (NS == 4 && j + 2 < nblk) wait_vm_lds<LOADS>();
      else wait_vm_lds<0>();
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      if (j + NS - 1 < nblk) issue_kv(j + NS - 1);
    }
    if (j >= nact) continue;
    const unsigned stj = stage_ptr(j);
    if (j + 1 < nact) {
      const unsigned stn = stage_ptr(j + 1);
      scores(stn, true);              // S_{j+1} - mu (matrix cores)
      if (j + 1 >= nfree) mask(j + 1);
      // value product of block j, sub-block by sub-block, interleaved with
      // the weights of block j+1 (the weights of sub-block kb are written
      // into pw[kb] only after block j's sub-block kb has been consumed)
      vec pn[NKB][2];
      float bn = 0.f;
      value_product(stj, 0);
      #pragma unroll
      for (int st = 0; st < 2; ++st) {
        floatx8 pf;
        #pragma unroll
        for (int t = 0; t < 8; ++t) pf[t] = __builtin_amdgcn_exp2f(s[0][8 * st + t]);
        pn[0][st] = Cvt<T>::eight(pf);
        bn = sum8(pn[0][st], bn);
      }
      value_product(stj, 1);
      #pragma unroll
      for (int st = 0; st < 2; ++st) {
        floatx8 pf;
        #pragma unroll
        for (int t = 0; t < 8; ++t) pf[t] = __builtin_amdgcn_exp2f(s[1][8 * st + t]);
        pn[1][st] = Cvt<T>::eight(pf);
        bn = sum8(pn[1][st], bn);
      }
      #pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        #pragma unroll
        for (int st = 0; st < 2; ++st) pw[kb][st] = pn[kb][st];
      if (__any(!(bn <= kLazyLimit))) {
        // rare: a weight of block j+1 exceeded 2^8 (or overflowed): redo it
        // from its raw scores with mu moved to the exact maximum
        scores(stn, false);
        if (j + 1 >= nfree) mask(j + 1);
        const float mu_new = fmaxf(mu, block_max());
        rescale(__builtin_amdgcn_exp2f(mu - mu_new));
        mu = mu_new;
        #pragma unroll
        for (int i = 0; i < 16; ++i) negmu[i] = -mu;
        bn = 0.f;
        weights(0, mu, bn);
        weights(1, mu, bn);
      }
      l_run += bn;
    } else {
      value_product(stj, 0);
      value_product(stj, 1);
    }
  }

  // ---- finalise: z / l into the concatenation ---------------------------------
  const float l_tot = half_sum(l_run);
  const float inv = 1.0f / l_tot;
  if (qi < p.n_q) {
    const size_t zbase = ((size_t)b * p.n_q + qi) * p.ldz + (size_t)r * DV;
    #pragma unroll
    for (int d = 0; d < C::NDV; ++d)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int e0 = d * 32 + 8 * a + 4 * g;
        store4(p.Z, p.out_dtype, zbase + e0, p.vec_z, DV - e0, o[d][4 * a] * inv,
               o[d][4 * a + 1] * inv, o[d][4 * a + 2] * inv, o[d][4 * a + 3] * inv);
      }
  }
}

}  // namespace mha
