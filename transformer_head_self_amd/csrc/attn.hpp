// Fused attention forward for gfx950 (one query tile per workgroup).
//
// Page "Stable summary of an attention key block", Definition: each query
// row keeps a summary (m, l, z) of the keys seen so far; the summary of the
// next key block is merged with the page's rule (the larger maximum becomes
// the shift, both sides are rescaled by exp of the old-minus-new maximum);
// at the end z is divided by l.  The empty state (no allowed key seen yet)
// is held as m = -inf, l = 0, z = 0, and the shift used for exponentials is
// forced to 0 while m is -inf, so the empty state merges as the identity.
// Review page "Multi-Head Attention", "The Complete Multi-Head Operation":
// scores are c * q_i . k_j, the mask is applied before the softmax, and the
// head result is written into its column block of the concatenation.
//
// Mapping onto the matrix cores (our design, not the pages'):
// * each wave owns 32 query rows; a workgroup of WAVES waves shares K/V
//   blocks of BN = 64 keys staged through LDS;
// * the score block is computed transposed, S^T = K Q^T, with a 32x32 MFMA:
//   lane l then holds 16 scores of query (l % 32) per 32-key sub-block, so a
//   row's maximum and sum need one exchange with the other half-wave only;
// * the value product is computed as O^T = V^T P^T: the transposed score
//   fragment is already in the B-operand layout of the next MFMA, and V is
//   staged transposed (d-major) in LDS so that each lane reads its keys
//   contiguously;
// * O^T leaves every lane with one query's output features, so the final
//   division by l and the concatenated store need no cross-lane traffic.
// Base-2 exponentials: scores are multiplied by c*log2(e), so
// 2^(x - m2) = e^(s - m) and l, z are the page's quantities exactly.
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace mha {

template <typename T, int DH, int DV, int WAVES>
struct AttnCfg {
  static constexpr int VEC = Elem<T>::VEC;
  static constexpr int BN = 64;                 // keys per block
  static constexpr int NT = 64 * WAVES;         // threads per workgroup
  static constexpr int QT = 32 * WAVES;         // queries per workgroup
  static constexpr int KCH = DH / (2 * VEC);    // k-chunks of the score MFMA
  static constexpr int NDV = DV / 32;           // 32-row blocks of V^T
  static constexpr int KPAD = DH + VEC;         // LDS row stride of K (elements)
  static constexpr int VPAD = BN + (sizeof(T) == 2 ? 4 : 4);  // LDS row stride of V^T
  static constexpr int K_CHUNKS = BN * DH / VEC;
  static constexpr int V_CHUNKS = BN * DV / VEC;
  static constexpr int K_PER_T = (K_CHUNKS + NT - 1) / NT;
  static constexpr int V_PER_T = (V_CHUNKS + NT - 1) / NT;
  static constexpr int LDS_BYTES = (BN * KPAD + DV * VPAD) * (int)sizeof(T);
  static_assert(DH % (2 * VEC) == 0, "DH must be a multiple of a k-chunk");
  static_assert(DV % 32 == 0, "DV must be a multiple of 32");
};

template <typename T, int DH, int DV, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void attn_fwd_kernel(AttnParams p) {
  typedef AttnCfg<T, DH, DV, WAVES> C;
  typedef typename Elem<T>::vec vec;
  constexpr int VEC = C::VEC;
  constexpr int BN = C::BN;

  __shared__ __attribute__((aligned(16))) T Ks[BN * C::KPAD];
  __shared__ __attribute__((aligned(16))) T Vt[DV * C::VPAD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;      // lane half
  const int l32 = lane & 31;

  // Workgroup -> (query tile, batch*head).  Query tiles outer, heads inner:
  // with round-robin dispatch over the 8 XCDs, every tile of one head lands
  // on the same XCD when B*h is a multiple of 8, so its K/V stay in that
  // XCD's L2.  Causal: longest tiles (most keys) first.
  const int BH = p.B * p.h;
  const int id = blockIdx.x;
  const int qt_rank = id / BH;
  const int bh = id - qt_rank * BH;
  const int qt = p.causal ? (p.num_q_tiles - 1 - qt_rank) : qt_rank;
  const int b = bh / p.h;
  const int r = bh - b * p.h;
  const int q0 = qt * C::QT;
  const int qw = q0 + wave * 32;
  const int qi = qw + l32;

  // Keys any row of this workgroup may use: [0, kend).
  int kvalid = p.n_k;
  if (p.key_len) kvalid = min(kvalid, p.key_len[b]);
  int kend = kvalid;
  if (p.causal) kend = min(kend, q0 + C::QT);
  const int nblk = kend > 0 ? (kend + BN - 1) / BN : 0;

  const T* Qb = reinterpret_cast<const T*>(p.Q) + (size_t)bh * p.n_q * p.ldq;
  const T* Kb = reinterpret_cast<const T*>(p.K) + (size_t)bh * p.n_k * p.ldk;
  const T* Vb = reinterpret_cast<const T*>(p.V) + (size_t)bh * p.n_k * p.ldv;
  const uint8_t* Gb = p.allowed ? p.allowed + (size_t)b * p.allowed_batch_stride : nullptr;
  const bool vq = p.vec_q, vk = p.vec_k, vv = p.vec_v;

  // This lane's query row as the B operand of S^T = K Q^T (registers, whole kernel).
  vec qf[C::KCH];
  #pragma unroll
  for (int c = 0; c < C::KCH; ++c)
    qf[c] = (qi < p.n_q) ? load_chunk<T>(Qb + (size_t)qi * p.ldq, c * 2 * VEC + g * VEC, p.d_h, vq)
                         : zero_vec<vec>();

  floatx16 o[C::NDV];
  #pragma unroll
  for (int d = 0; d < C::NDV; ++d)
    #pragma unroll
    for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
  float m_run = -INFINITY;  // running maximum (base-2 units)
  float l_run = 0.f;        // this half-wave's part of the running normaliser

  vec kreg[C::K_PER_T];
  vec vreg[C::V_PER_T];

  auto load_kv = [&](int blk) {
    const int k0 = blk * BN;
    #pragma unroll
    for (int t = 0; t < C::K_PER_T; ++t) {
      const int ci = tid + t * C::NT;
      const int row = ci / (DH / VEC);
      const int cc = ci - row * (DH / VEC);
      const int key = k0 + row;
      kreg[t] = (ci < C::K_CHUNKS && key < p.n_k)
                    ? load_chunk<T>(Kb + (size_t)key * p.ldk, cc * VEC, p.d_h, vk)
                    : zero_vec<vec>();
    }
    #pragma unroll
    for (int t = 0; t < C::V_PER_T; ++t) {
      const int ci = tid + t * C::NT;
      const int cc = ci / BN;          // consecutive threads take consecutive keys,
      const int row = ci - cc * BN;    // so the transposed LDS stores are contiguous
      const int key = k0 + row;
      vreg[t] = (ci < C::V_CHUNKS && key < p.n_k)
                    ? load_chunk<T>(Vb + (size_t)key * p.ldv, cc * VEC, p.d_vh, vv)
                    : zero_vec<vec>();
    }
  };
  auto store_kv = [&]() {
    #pragma unroll
    for (int t = 0; t < C::K_PER_T; ++t) {
      const int ci = tid + t * C::NT;
      if (ci < C::K_CHUNKS) {
        const int row = ci / (DH / VEC);
        const int cc = ci - row * (DH / VEC);
        *reinterpret_cast<vec*>(&Ks[row * C::KPAD + cc * VEC]) = kreg[t];
      }
    }
    #pragma unroll
    for (int t = 0; t < C::V_PER_T; ++t) {
      const int ci = tid + t * C::NT;
      if (ci < C::V_CHUNKS) {
        const int cc = ci / BN;
        const int row = ci - cc * BN;
        #pragma unroll
        for (int e = 0; e < VEC; ++e) Vt[(cc * VEC + e) * C::VPAD + row] = vreg[t][e];
      }
    }
  };

  if (nblk > 0) load_kv(0);

  for (int blk = 0; blk < nblk; ++blk) {
    __syncthreads();  // every wave is done reading the previous block
    store_kv();
    __syncthreads();
    if (blk + 1 < nblk) load_kv(blk + 1);  // in flight while this block computes

    const int k0 = blk * BN;
    // A wave whose rows all precede this block's first key (causal) sees an
    // empty key set here: its summary is the empty state, a no-op merge.
    const bool active = (qw < p.n_q) && !(p.causal && k0 > qw + 31);
    if (!active) continue;

    // ---- scores S^T (two 32-key sub-blocks) --------------------------------
    floatx16 s[2];
    #pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      #pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
      #pragma unroll
      for (int c = 0; c < C::KCH; ++c) {
        const vec kf = *reinterpret_cast<const vec*>(
            &Ks[(kb * 32 + l32) * C::KPAD + c * 2 * VEC + g * VEC]);
        mfma_chunk(s[kb], kf, qf[c]);
      }
    }

    // ---- scale, mask, block maximum -----------------------------------------
    const bool need_mask = (k0 + BN > kvalid) || (p.causal && k0 + BN - 1 > qw) || Gb != nullptr;
    float mx = -INFINITY;
    #pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      #pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[kb][i] * p.scale_log2;
        if (need_mask) {
          const int j = k0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          bool ok = j < kvalid;
          if (p.causal) ok = ok && (j <= qi);
          if (Gb != nullptr && ok) ok = qi < p.n_q && Gb[(size_t)qi * p.n_k + j] != 0;
          x = ok ? x : -INFINITY;
        }
        s[kb][i] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, wave_xor32(mx));

    // ---- merge: new shift, rescale the running summary ----------------------
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float lsum = 0.f;
    #pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      #pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pe = __builtin_amdgcn_exp2f(s[kb][i] - m_use);
        s[kb][i] = pe;
        lsum += pe;
      }
    l_run = l_run * alpha + lsum;
    #pragma unroll
    for (int d = 0; d < C::NDV; ++d)
      #pragma unroll
      for (int i = 0; i < 16; ++i) o[d][i] *= alpha;

    // ---- z += P V  (as O^T += V^T P^T) -------------------------------------
    #pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (sizeof(T) == 2) {
        #pragma unroll
        for (int st = 0; st < 2; ++st) {
          bf16x8 pb;
          #pragma unroll
          for (int t = 0; t < 8; t += 2) {
            floatx2 f2 = {s[kb][8 * st + t], s[kb][8 * st + t + 1]};
            bf16x2 b2 = __builtin_convertvector(f2, bf16x2);
            pb[t] = b2.x;
            pb[t + 1] = b2.y;
          }
          #pragma unroll
          for (int d = 0; d < C::NDV; ++d) {
            const T* vrow = &Vt[(d * 32 + l32) * C::VPAD + kb * 32 + 16 * st + 4 * g];
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + 8);
            const bf16x8 va = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            mfma_chunk(o[d], va, pb);
          }
        }
      } else {
        #pragma unroll
        for (int a = 0; a < 4; ++a) {
          const floatx4 pf = {s[kb][4 * a], s[kb][4 * a + 1], s[kb][4 * a + 2], s[kb][4 * a + 3]};
          #pragma unroll
          for (int d = 0; d < C::NDV; ++d) {
            const floatx4 va = *reinterpret_cast<const floatx4*>(
                &Vt[(d * 32 + l32) * C::VPAD + kb * 32 + 8 * a + 4 * g]);
            mfma_chunk(o[d], va, pf);
          }
        }
      }
    }
  }

  // ---- finalise: z / l, store into the concatenation --------------------------
  const float l_tot = l_run + wave_xor32(l_run);
  const float inv = 1.0f / l_tot;
  if (qi < p.n_q) {
    const size_t zbase = ((size_t)b * p.n_q + qi) * p.ldz + (size_t)r * p.d_vh;
    #pragma unroll
    for (int d = 0; d < C::NDV; ++d) {
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int e0 = d * 32 + 8 * a + 4 * g;
        store4(p.Z, p.out_dtype, zbase + e0, p.vec_z, p.d_vh - e0, o[d][4 * a] * inv,
               o[d][4 * a + 1] * inv, o[d][4 * a + 2] * inv, o[d][4 * a + 3] * inv);
      }
    }
    if (g == 0) {
      const size_t ri = (size_t)bh * p.n_q + qi;
      if (p.row_m) p.row_m[ri] = (m_run == -INFINITY) ? -INFINITY : m_run * kLn2;
      if (p.row_l) p.row_l[ri] = l_tot;
    }
  }
}

}  // namespace mha
