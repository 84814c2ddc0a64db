// Key-partition kernel for a few query rows against many keys (decoding),
// gfx950, 2-byte elements.
//
// Same results as the split form of attn_fwd_kernel: for each key partition
// of each (item, head) it writes the rows' partial summaries (m, l, z) of
// page "Stable summary of an attention key block", Definition, in base-2
// units; the merge kernel combines them.  With one to four query rows the
// 32-row matrix-core tiles would be almost all padding, and the step is
// bound by reading the key/value cache once, so this kernel uses the vector
// ALU instead (our design):
// * a group of G lanes holds one cached key row and its value row, 16 bytes
//   per lane (G = 4, 8 or 16 for rows of up to 32, 64 or 128 elements); a
//   wave covers 64 / G keys per step and each lane streams its own 16-byte
//   chunks, so a wave's loads are contiguous runs of whole rows; the cache is
//   read once, with non-temporal loads (measured 11 % faster);
// * a score is the lane's 8-term dot product summed over the group with DPP
//   row exchanges (no LDS);
// * each group keeps its own running summary per query row, merged with the
//   page's rule: U keys at a time, the shift moves to the largest score seen
//   and both sides are rescaled by 2^(old - new);
// * at the end the groups of a wave merge by lane exchanges, the four waves
//   through LDS, and the partition's summary is written.
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace mha {

// Sum over aligned groups of G lanes (G = 4, 8, 16) with DPP row moves:
// xor 1, xor 2 (quad permutes), then the half-row and row mirrors, which pair
// each lane with one in the other half of its 8- or 16-lane group.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  int xi = __builtin_bit_cast(int, x);
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, xi, 0xB1, 0xF, 0xF, false));
  xi = __builtin_bit_cast(int, x);
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, xi, 0x4E, 0xF, 0xF, false));
  if constexpr (G >= 8) {
    xi = __builtin_bit_cast(int, x);
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, xi, 0x141, 0xF, 0xF, false));
  }
  if constexpr (G >= 16) {
    xi = __builtin_bit_cast(int, x);
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, xi, 0x140, 0xF, 0xF, false));
  }
  return x;
}

// Merge summary (m2, l2, z2) into (m, l, z) (base 2; the empty state m = -inf
// is the identity).
template <int E>
__device__ __forceinline__ void merge_summary(float& m, float& l, float (&z)[E], float m2, float l2,
                                              const float (&z2)[E]) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;                 // both empty
  const float a = __builtin_amdgcn_exp2f(m - mn), c = __builtin_amdgcn_exp2f(m2 - mn);
  l = l * a + l2 * c;
  #pragma unroll
  for (int e = 0; e < E; ++e) z[e] = z[e] * a + z2[e] * c;
  m = mn;
}

template <typename T, int G, int NQ>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnParams p) {
  typedef typename Elem<T>::vec vec;
  constexpr int KPW = 64 / G;          // keys per wave step
  constexpr int U = 4;                 // keys per group per iteration
  constexpr int STRIDE = 4 * KPW;      // keys per workgroup step
  __shared__ float red_m[4][NQ], red_l[4][NQ];
  __shared__ float red_z[4][NQ][G * 8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane / G, gl = lane % G;
  const int sp = (int)(blockIdx.x % (unsigned)p.splits);
  const int bh = (int)(blockIdx.x / (unsigned)p.splits);
  const int b = bh / p.h;
  int kvalid = p.n_k;
  if (p.key_len) kvalid = min(kvalid, p.key_len[b]);
  const int kbeg = sp * p.split_keys;
  int kend = min(kvalid, kbeg + p.split_keys);
  if (p.causal) kend = min(kend, p.n_q);      // key j <= query i <= n_q - 1

  const T* Qb = reinterpret_cast<const T*>(p.Q) + (size_t)bh * p.n_q * p.ldq;
  const T* Kb = reinterpret_cast<const T*>(p.K) + (size_t)bh * p.n_k * p.ldk;
  const T* Vb = reinterpret_cast<const T*>(p.V) + (size_t)bh * p.n_k * p.ldv;
  const uint8_t* Gm = p.allowed ? p.allowed + (size_t)b * p.allowed_batch_stride : nullptr;
  const float* Ab = p.add ? p.add + (size_t)b * p.add_batch_stride : nullptr;
  const int nq = min(p.n_q, NQ);
  const bool kin = gl * 8 < p.d_h, vin = gl * 8 < p.d_vh;   // this lane's chunks exist

  // query chunks, scaled by c log2(e) (scores then come out in base 2)
  float q[NQ][8];
  #pragma unroll
  for (int i = 0; i < NQ; ++i) {
    vec qc = zero_vec<vec>();
    if (i < nq && kin) qc = *reinterpret_cast<const vec*>(Qb + (size_t)i * p.ldq + gl * 8);
    #pragma unroll
    for (int e = 0; e < 8; ++e) q[i][e] = (float)qc[e] * p.scale_log2;
  }
  float m[NQ], l[NQ], z[NQ][8];
  #pragma unroll
  for (int i = 0; i < NQ; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
    #pragma unroll
    for (int e = 0; e < 8; ++e) z[i][e] = 0.f;
  }
  const bool general = p.causal || Gm != nullptr || Ab != nullptr;

  for (int k0 = kbeg + wave * KPW + grp; k0 < kend; k0 += U * STRIDE) {
    vec kc[U], vc[U];
    #pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = min(k0 + u * STRIDE, kend - 1);   // past the end: a valid row, masked
      kc[u] = kin ? __builtin_nontemporal_load(reinterpret_cast<const vec*>(Kb + (size_t)key * p.ldk + gl * 8)) : zero_vec<vec>();
      vc[u] = vin ? __builtin_nontemporal_load(reinterpret_cast<const vec*>(Vb + (size_t)key * p.ldv + gl * 8)) : zero_vec<vec>();
    }
    #pragma unroll
    for (int i = 0; i < NQ; ++i) {
      if (i >= nq) break;
      float s[U];
      float mx = -INFINITY;
      #pragma unroll
      for (int u = 0; u < U; ++u) {
        float d = 0.f;
        #pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(q[i][e], (float)kc[u][e], d);
        d = group_sum<G>(d);
        const int key = k0 + u * STRIDE;
        bool ok = key < kend;
        if (general && ok) {
          if (p.causal && key > i) ok = false;
          if (Gm != nullptr && Gm[(size_t)i * p.n_k + key] == 0) ok = false;
          if (Ab != nullptr && ok) d = fmaf(Ab[(size_t)i * p.n_k + key], kLog2e, d);
        }
        s[u] = ok ? d : -INFINITY;
        mx = fmaxf(mx, s[u]);
      }
      const float mn = fmaxf(m[i], mx);
      if (mn == -INFINITY) continue;                     // nothing allowed yet
      const float a = __builtin_amdgcn_exp2f(m[i] - mn);
      m[i] = mn;
      l[i] *= a;
      #pragma unroll
      for (int e = 0; e < 8; ++e) z[i][e] *= a;
      #pragma unroll
      for (int u = 0; u < U; ++u) {
        const float w = (s[u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[u] - mn);
        l[i] += w;
        #pragma unroll
        for (int e = 0; e < 8; ++e) z[i][e] = fmaf(w, (float)vc[u][e], z[i][e]);
      }
    }
  }

  // groups of a wave: lanes gl of groups grp and grp ^ step exchange and merge
  #pragma unroll
  for (int st = G; st < 64; st <<= 1) {
    #pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const float m2 = __shfl_xor(m[i], st, 64);
      const float l2 = __shfl_xor(l[i], st, 64);
      float z2[8];
      #pragma unroll
      for (int e = 0; e < 8; ++e) z2[e] = __shfl_xor(z[i][e], st, 64);
      merge_summary<8>(m[i], l[i], z[i], m2, l2, z2);
    }
  }
  // waves: through LDS, merged by wave 0
  if (lane < G) {
    #pragma unroll
    for (int i = 0; i < NQ; ++i) {
      if (lane == 0) {
        red_m[wave][i] = m[i];
        red_l[wave][i] = l[i];
      }
      #pragma unroll
      for (int e = 0; e < 8; ++e) red_z[wave][i][lane * 8 + e] = z[i][e];
    }
  }
  __syncthreads();
  if (wave == 0 && lane < G) {
    #pragma unroll
    for (int i = 0; i < NQ; ++i) {
      #pragma unroll
      for (int w = 1; w < 4; ++w) {
        float z2[8];
        #pragma unroll
        for (int e = 0; e < 8; ++e) z2[e] = red_z[w][i][lane * 8 + e];
        merge_summary<8>(m[i], l[i], z[i], red_m[w][i], red_l[w][i], z2);
      }
      if (i < nq) {
        const size_t pr = ((size_t)sp * p.B * p.h + bh) * p.n_q + i;
        #pragma unroll
        for (int e = 0; e < 8; ++e)
          if (lane * 8 + e < p.d_vh) p.part_z[pr * p.d_vh + lane * 8 + e] = z[i][e];
        if (lane == 0) {
          p.part_m[pr] = m[i];
          p.part_l[pr] = l[i];
        }
      }
    }
  }
}

}  // namespace mha
