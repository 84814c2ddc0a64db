// Backward pass of the fused attention core for gfx950 (2-byte elements,
// fp32 accumulation).
//
// The pages define the forward pass only; the gradients follow from it by
// calculus.  For one head with scores S = c Q K^T (+ M), weights A = the
// masked row softmax of S and output Z = A V, and an upstream gradient dZ:
//   dV = A^T dZ,   dA = dZ V^T,   dS = A o (dA - D),  D_i = sum_e dZ_ie Z_ie,
//   dQ = c dS K,   dK = c dS^T Q.
// The weights are recomputed block by block from the forward's row
// statistics: page "Stable summary of an attention key block", Definition,
// gives A_ij = e^(s_ij - m_i) / l_i for the final (m, l) of row i, so no
// n_q x n_k matrix is stored.  Here A_ij = 2^(s_ij c log2(e) - L_i) with
// L_i = m_i log2(e) + log2(l_i) prepared once per row (attn_bwd_prep_kernel,
// which also forms D_i).
//
// Mapping onto the matrix cores (ours), with the 32x32x16 MFMA whose result
// acc[i] holds row 8 (i/4) + 4 g + (i%4), column l % 32:
// * attn_bwd_kv_kernel: a wave owns 32 keys; query tiles of 64 rows of Q and
//   dZ stream through LDS.  S = Q K^T and dA = dZ V^T put one key per lane
//   (K and V rows are the B operands, held in registers), so A and dS come
//   out in the B-operand layout of dV^T += dZ^T A and dK^T += Q^T dS, whose
//   A operands (dZ^T, Q^T) are read from row-major LDS tiles with the
//   transposing load, exactly as the forward reads V^T.
// * attn_bwd_q_kernel: a wave owns 32 queries, key tiles stream through LDS
//   (the forward's structure): S^T = K Q^T and dA^T = V dZ^T put one query
//   per lane, and dQ^T += K^T dS^T reads K^T with the transposing load.
// Two kernels instead of one with atomic dQ updates: the sums are formed in
// a fixed order, so runs are deterministic.
#pragma once

#include "common.hpp"
#include "internal.hpp"
#include "lds_dma.hpp"

namespace mha {

template <int DH, int DV>
struct BwdCfg {
  static constexpr int WAVES = 4;
  static constexpr int NT = 64 * WAVES;
  static constexpr int VEC = 8;              // 2-byte elements per 16-byte chunk
  static constexpr int BR = 64;              // rows of a streamed tile
  static constexpr int KCH = DH / 16;        // MFMA k-chunks over d_h
  static constexpr int VCH = DV / 16;        // MFMA k-chunks over d_vh
  static constexpr int NDH = DH / 32;        // 32-row blocks of dK^T / dQ^T
  static constexpr int NDV = DV / 32;        // 32-row blocks of dV^T
  static constexpr int HROW = DH + 8;        // LDS row strides (elements): 16 bytes of
  static constexpr int VROW = DV + 8;        // padding stagger the rows over the banks
  static constexpr int HTILE = BR * HROW, VTILE = BR * VROW;
  static constexpr int H_PER_T = (BR * DH / VEC + NT - 1) / NT;
  static constexpr int V_PER_T = (BR * DV / VEC + NT - 1) / NT;
  // waves per SIMD the dK/dV kernel's registers must allow: two (at most
  // 256 VGPRs) unless its accumulators and operand rows need more
  static constexpr int KV_OCC = (DH + DV <= 160) ? 2 : 1;
  static_assert(DH % 32 == 0 && DV % 32 == 0, "head widths are multiples of 32");
};

// Eight consecutive elements of a row of element type `dtype` (fp32, bf16
// or fp16) at `base + off`, columns col..col+7 of `ncols` valid ones (zero
// past the end), rounded to T (nearest even).
template <typename T>
__device__ __forceinline__ typename Elem<T>::vec load8_as(const void* base, int dtype, size_t off,
                                                          int col, int ncols, bool vec_ok) {
  typedef typename Elem<T>::vec V;
  if (dtype == kF32) {
    const float* row = reinterpret_cast<const float*>(base) + off;
    floatx8 f;
    if (vec_ok && col + 8 <= ncols) {
      const floatx4 a = *reinterpret_cast<const floatx4*>(row + col);
      const floatx4 b = *reinterpret_cast<const floatx4*>(row + col + 4);
      f = floatx8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
      #pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = (col + e < ncols) ? row[col + e] : 0.f;
    }
    return __builtin_convertvector(f, V);
  } else if (dtype == kBF16) {
    return convert_chunk<T, bf16>(
        load_chunk<bf16>(reinterpret_cast<const bf16*>(base) + off, col, ncols, vec_ok));
  } else {
    return convert_chunk<T, f16>(
        load_chunk<f16>(reinterpret_cast<const f16*>(base) + off, col, ncols, vec_ok));
  }
}

__device__ __forceinline__ float load1_as(const void* base, int dtype, size_t idx) {
  if (dtype == kF32) return reinterpret_cast<const float*>(base)[idx];
  if (dtype == kBF16) return (float)reinterpret_cast<const bf16*>(base)[idx];
  return (float)reinterpret_cast<const f16*>(base)[idx];
}

// Per row and head: D = sum_e dZ Z, and L = m log2(e) + log2(l) (+inf for a
// row without allowed keys, whose weights are then all 0).  dZ enters D
// rounded to the element type, as it enters the products dA = dZ V^T: D then
// matches the row sum sum_j A_ij dA_ij of the rounded dZ, and dA - D carries
// no rounding mismatch into the cancellation between the two.
__device__ __forceinline__ void bwd_row_terms(const AttnBwdParams& p, int b, int r, int qi,
                                              float dsum) {
  const size_t idx = ((size_t)b * p.h + r) * p.n_q + qi;
  p.dsum[idx] = dsum;
  const float m = p.row_m[idx], l = p.row_l[idx];
  p.lse2[idx] = (l > 0.f && m != -INFINITY) ? fmaf(m, kLog2e, __log2f(l)) : INFINITY;
}

// x rounded to the heads' element type (fp32 heads: unchanged).
__device__ __forceinline__ float round_as(float x, int elem_dtype) {
  if (elem_dtype == kF32) return x;
  return elem_dtype == kBF16 ? (float)(bf16)x : (float)(f16)x;
}

// General form: one wave per (query row, head); lanes take elements e and
// e + 64, and the wave sums its lanes.
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(AttnBwdParams p) {
  const int lane = threadIdx.x & 63;
  const size_t pair = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (b*n_q + q)*h + r
  const size_t npairs = (size_t)p.B * p.n_q * p.h;
  if (pair >= npairs) return;                                        // whole wave
  const size_t row = pair / p.h;                                     // b*n_q + q
  const int r = (int)(pair - row * p.h);
  const int b = (int)(row / p.n_q);
  const size_t off = row * p.ldz + (size_t)r * p.d_vh;
  float acc = 0.f;
  for (int e = lane; e < p.d_vh; e += 64)
    acc = fmaf(round_as(load1_as(p.dZ, p.z_dtype, off + e), p.elem_dtype),
               load1_as(p.Z, p.z_dtype, off + e), acc);
  #pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (lane == 0) bwd_row_terms(p, b, r, (int)(row - (size_t)b * p.n_q), acc);
}

// Vector form (2-byte Z and dZ, d_vh in {32, 64, 128}, 16-byte aligned
// rows): the rows of the concatenation [B*n_q, h*d_vh] are read as 16-byte
// chunks by consecutive threads; the CPH = d_vh / 8 consecutive lanes that
// hold one head's chunks of a row sum them with lane exchanges.
template <typename TZ, int CPH>
__global__ __launch_bounds__(256) void attn_bwd_prep_vec_kernel(AttnBwdParams p) {
  typedef typename Elem<TZ>::vec vec;
  const size_t chunks = (size_t)p.B * p.n_q * p.ldz / 8;
  const size_t ci = (size_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = ci < chunks;
  float acc = 0.f;
  size_t row = 0;
  int cr = 0;
  if (live) {
    const vec dz = reinterpret_cast<const vec*>(p.dZ)[ci];
    const vec z = reinterpret_cast<const vec*>(p.Z)[ci];
    #pragma unroll
    for (int t = 0; t < 8; ++t) acc = fmaf(round_as((float)dz[t], p.elem_dtype), (float)z[t], acc);
    const size_t per_row = (size_t)p.ldz / 8;
    row = ci / per_row;
    cr = (int)(ci - row * per_row);
  }
  #pragma unroll
  for (int m = CPH / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (live && cr % CPH == 0) {
    const int b = (int)(row / p.n_q);
    bwd_row_terms(p, b, cr / CPH, (int)(row - (size_t)b * p.n_q), acc);
  }
}

// Stage one 64-row tile of a row-major [rows x ncols] array (row stride ld,
// element type dtype) into LDS rows of ROW elements, rounded to T; rows past
// `nrows` and columns past `ncols` are zero.
template <typename T, int D, int ROW, int PER_T, int NT>
struct TileStager {
  typedef typename Elem<T>::vec vec;
  vec reg[PER_T];
  __device__ __forceinline__ void load(const void* base, int dtype, size_t row0_off, size_t ld,
                                       int r0, int nrows, int ncols, bool vec_ok, int tid) {
    #pragma unroll
    for (int t = 0; t < PER_T; ++t) {
      const int ci = tid + t * NT;
      if ((64 * D / 8) % NT != 0 && ci >= 64 * D / 8) continue;
      const int row = ci / (D / 8), col = (ci - row * (D / 8)) * 8;
      reg[t] = (r0 + row < nrows)
                   ? load8_as<T>(base, dtype, row0_off + (size_t)(r0 + row) * ld, col, ncols, vec_ok)
                   : zero_vec<vec>();
    }
  }
  __device__ __forceinline__ void store(T* tile, int tid) const {
    #pragma unroll
    for (int t = 0; t < PER_T; ++t) {
      const int ci = tid + t * NT;
      if ((64 * D / 8) % NT != 0 && ci >= 64 * D / 8) continue;
      const int row = ci / (D / 8), col = (ci - row * (D / 8)) * 8;
      *reinterpret_cast<vec*>(&tile[row * ROW + col]) = reg[t];
    }
  }
};

// Is key `key` allowed for query `q` of item b (general rules; n_q, n_k and
// key padding bounds included)?
__device__ __forceinline__ bool bwd_allowed(const AttnBwdParams& p, const uint8_t* G, int q,
                                            int key, int kvalid) {
  if (q >= p.n_q || key >= kvalid) return false;
  if (p.causal && key > q) return false;
  if (G != nullptr && G[(size_t)q * p.n_k + key] == 0) return false;
  return true;
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (128 keys, b*h + r); a wave owns 32 keys.
// ---------------------------------------------------------------------------
template <typename T, int DH, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BwdCfg<DH, DV>::KV_OCC, 2)))
void attn_bwd_kv_kernel(AttnBwdParams p) {
  typedef BwdCfg<DH, DV> C;
  typedef typename Elem<T>::vec vec;
  typedef typename Elem<T>::vec4 vec4;
  __shared__ __attribute__((aligned(16))) T Qs[2][C::HTILE];
  __shared__ __attribute__((aligned(16))) T Zs[2][C::VTILE];
  __shared__ float Ls[2][C::BR], Ds[2][C::BR];
  constexpr int tdt = __is_same(T, bf16) ? kBF16 : kF16;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int BH = p.B * p.h;
  const int kt = blockIdx.x / BH;             // key tile (earliest keys first: most queries)
  const int bh = blockIdx.x - kt * BH;
  const int b = bh / p.h, r = bh - b * p.h;
  const int k0 = kt * 128, k0w = k0 + 32 * wave;
  const int key = k0w + l32;                  // this lane's key
  int kvalid = p.n_k;
  if (p.key_len) kvalid = min(kvalid, p.key_len[b]);

  const T* Qb = reinterpret_cast<const T*>(p.Q) + (size_t)bh * p.n_q * p.d_h;
  const T* Kb = reinterpret_cast<const T*>(p.K) + (size_t)bh * p.n_k * p.d_h;
  const T* Vb = reinterpret_cast<const T*>(p.V) + (size_t)bh * p.n_k * p.d_vh;
  const size_t zoff = (size_t)b * p.n_q * p.ldz + (size_t)r * p.d_vh;   // row 0 of this head
  const uint8_t* G = p.allowed ? p.allowed + (size_t)b * p.allowed_batch_stride : nullptr;
  const float* M = p.add ? p.add + (size_t)b * p.add_batch_stride : nullptr;
  const float* lse = p.lse2 + (size_t)bh * p.n_q;
  const float* dsm = p.dsum + (size_t)bh * p.n_q;

  // this lane's key row of K and V as B operands (k-chunk c: elements
  // 16 c + 8 g .. +7); keys past n_k read as zero
  vec kf[C::KCH], vf[C::VCH];
  #pragma unroll
  for (int c = 0; c < C::KCH; ++c)
    kf[c] = key < p.n_k ? load_chunk<T>(Kb + (size_t)key * p.d_h, 16 * c + 8 * g, p.d_h, p.vec_k)
                        : zero_vec<vec>();
  #pragma unroll
  for (int c = 0; c < C::VCH; ++c)
    vf[c] = key < p.n_k ? load_chunk<T>(Vb + (size_t)key * p.d_vh, 16 * c + 8 * g, p.d_vh, p.vec_v)
                        : zero_vec<vec>();

  floatx16 dk[C::NDH], dv[C::NDV];
  #pragma unroll
  for (int d = 0; d < C::NDH; ++d)
    #pragma unroll
    for (int i = 0; i < 16; ++i) dk[d][i] = 0.f;
  #pragma unroll
  for (int d = 0; d < C::NDV; ++d)
    #pragma unroll
    for (int i = 0; i < 16; ++i) dv[d][i] = 0.f;

  // query tiles that can reach this key tile: causal needs q >= key
  const int qb0 = (p.causal ? k0 : 0) / C::BR;
  const int nqb = (k0 < kvalid) ? (p.n_q + C::BR - 1) / C::BR : qb0;   // padded keys only: none

  TileStager<T, DH, C::HROW, C::H_PER_T, C::NT> qst;
  TileStager<T, DV, C::VROW, C::V_PER_T, C::NT> zst;
  float lreg = 0.f, dreg = 0.f;
  auto load_tile = [&](int qb) {
    const int q0 = qb * C::BR;
    qst.load(Qb, tdt, 0, p.d_h, q0, p.n_q, p.d_h, p.vec_q, tid);
    zst.load(p.dZ, p.z_dtype, zoff, p.ldz, q0, p.n_q, p.d_vh, p.vec_z, tid);
    if (tid < C::BR) {
      const int q = q0 + tid;
      lreg = q < p.n_q ? lse[q] : INFINITY;
      dreg = q < p.n_q ? dsm[q] : 0.f;
    }
  };
  auto store_tile = [&](int buf) {
    qst.store(Qs[buf], tid);
    zst.store(Zs[buf], tid);
    if (tid < C::BR) {
      Ls[buf][tid] = lreg;
      Ds[buf][tid] = dreg;
    }
  };

  if (nqb > qb0) {
    load_tile(qb0);
    store_tile(0);
  }
  __syncthreads();
  if (nqb > qb0 + 1) load_tile(qb0 + 1);

  const int srow = 4 * g + ((lane & 15) >> 2);
  const int scol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const float cs = p.scale_log2;

  for (int qb = qb0; qb < nqb; ++qb) {
    const int cur = (qb - qb0) & 1;
    const T* qs = Qs[cur];
    const T* zs = Zs[cur];
    const int q0 = qb * C::BR;
    #pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int qs0 = q0 + 32 * sb;
      // whole sub-block before this wave's first key (causal), or every key
      // of the wave padded: nothing to add
      if ((p.causal && qs0 + 31 < k0w) || k0w >= kvalid || qs0 >= p.n_q) continue;
      floatx16 sacc, dpacc;
      #pragma unroll
      for (int i = 0; i < 16; ++i) {
        sacc[i] = 0.f;
        dpacc[i] = 0.f;
      }
      // S = Q K^T (lane: key l32; registers: queries), dA = dZ V^T
      #pragma unroll
      for (int c = 0; c < C::KCH; ++c) {
        const vec qa = *reinterpret_cast<const vec*>(&qs[(32 * sb + l32) * C::HROW + 16 * c + 8 * g]);
        mfma_chunk(sacc, qa, kf[c]);
      }
      #pragma unroll
      for (int c = 0; c < C::VCH; ++c) {
        const vec za = *reinterpret_cast<const vec*>(&zs[(32 * sb + l32) * C::VROW + 16 * c + 8 * g]);
        mfma_chunk(dpacc, za, vf[c]);
      }
      // A and dS; query of slot i: q0 + 32 sb + 8 (i/4) + 4 g + i%4
      const bool need_mask = (p.causal && qs0 < k0w + 31) || (k0w + 31 >= kvalid) ||
                             (qs0 + 31 >= p.n_q) || G != nullptr || M != nullptr;
      // exponent of each weight; a forbidden score's becomes -inf (weight
      // exactly 0) without a branch per score
      if (need_mask) {
        #pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ql = 32 * sb + 8 * (i >> 2) + 4 * g + (i & 3);
          const int q = q0 + ql;
          const bool ok = bwd_allowed(p, G, q, key, kvalid);
          float x;
          if (M != nullptr) {
            x = sacc[i] * cs;
            if (ok) x = fmaf(M[(size_t)q * p.n_k + key], kLog2e, x);
            x -= Ls[cur][ql];
          } else {
            x = fmaf(sacc[i], cs, -Ls[cur][ql]);
          }
          sacc[i] = ok ? x : -INFINITY;
        }
      } else {
        #pragma unroll
        for (int i = 0; i < 16; ++i)
          sacc[i] = fmaf(sacc[i], cs, -Ls[cur][32 * sb + 8 * (i >> 2) + 4 * g + (i & 3)]);
      }
      #pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ql = 32 * sb + 8 * (i >> 2) + 4 * g + (i & 3);
        const float a = __builtin_amdgcn_exp2f(sacc[i]);
        sacc[i] = a;
        dpacc[i] = a * (dpacc[i] - Ds[cur][ql]);
      }
      // dV^T += dZ^T A and dK^T += Q^T dS; slot t of chunk st is query
      // 16 st + 4 g + t (t < 4) or 16 st + 8 + 4 g + (t - 4), as in the
      // transposing read below
      #pragma unroll
      for (int st = 0; st < 2; ++st) {
        floatx8 af, sf;
        #pragma unroll
        for (int t = 0; t < 8; ++t) {
          af[t] = sacc[8 * st + t];
          sf[t] = dpacc[8 * st + t];
        }
        const vec ab = Cvt<T>::eight(af);
        const vec sbv = Cvt<T>::eight(sf);
        #pragma unroll
        for (int d = 0; d < C::NDV; ++d) {
          const T* v0 = &zs[(32 * sb + 16 * st + srow) * C::VROW + d * 32 + scol];
          const vec4 lo = lds_read_tr4<T>(v0);
          const vec4 hi = lds_read_tr4<T>(v0 + 8 * C::VROW);
          const vec za = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          mfma_chunk(dv[d], za, ab);
        }
        #pragma unroll
        for (int d = 0; d < C::NDH; ++d) {
          const T* q0p = &qs[(32 * sb + 16 * st + srow) * C::HROW + d * 32 + scol];
          const vec4 lo = lds_read_tr4<T>(q0p);
          const vec4 hi = lds_read_tr4<T>(q0p + 8 * C::HROW);
          const vec qa = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          mfma_chunk(dk[d], qa, sbv);
        }
      }
    }
    if (qb + 1 < nqb) store_tile(cur ^ 1);
    __syncthreads();
    if (qb + 2 < nqb) load_tile(qb + 2);
  }

  // dK = c (dK^T)^T, dV = (dV^T)^T: lane writes its key's row
  if (key < p.n_k) {
    // head-major [B, h, n_k, d] or concatenated [B, n_k, h*d]
    const size_t krow = p.grad_concat ? ((size_t)b * p.n_k + key) * p.h + r
                                      : (size_t)bh * p.n_k + key;
    const size_t kro = krow * p.d_h;
    const size_t vro = krow * p.d_vh;
    #pragma unroll
    for (int d = 0; d < C::NDH; ++d)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int e0 = d * 32 + 8 * a + 4 * g;
        store4(p.dK, p.g_dtype, kro + e0, p.vec_dk, p.d_h - e0, dk[d][4 * a] * p.scale,
               dk[d][4 * a + 1] * p.scale, dk[d][4 * a + 2] * p.scale, dk[d][4 * a + 3] * p.scale);
      }
    #pragma unroll
    for (int d = 0; d < C::NDV; ++d)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int e0 = d * 32 + 8 * a + 4 * g;
        store4(p.dV, p.g_dtype, vro + e0, p.vec_dv, p.d_vh - e0, dv[d][4 * a], dv[d][4 * a + 1],
               dv[d][4 * a + 2], dv[d][4 * a + 3]);
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV with direct-to-LDS tiles (2-byte Q and dZ of exactly DH / DV
// columns, 16-byte aligned rows, n_q a multiple of 4).  Same products, order
// of summation and results as attn_bwd_kv_kernel; the 64-row Q and dZ tiles
// and the rows' L and D move from global memory straight into LDS (three
// stages in flight) instead of through registers.
//
// Each tile is read with two patterns: 16-byte row reads (the A operand of
// S = Q K^T and dA = dZ V^T) and transposing reads (dZ^T, Q^T).  Rows are
// stored unpadded with chunk c of row r in slot c ^ bwd_swizzle(r); with the
// bank line of 256 bytes, h = r / (256 / RB) the bank line of row r and q the
// number of 64-byte quarters in a row, bwd_swizzle = 4 (h % q) + (h / q) % 4:
// 16 consecutive rows at one chunk fall in 16 distinct 16-byte bank groups,
// and the four rows a transposing read touches at one column fall in four
// distinct 64-byte quarters (checked exhaustively on the CPU).
// ---------------------------------------------------------------------------
template <int RB>
__device__ __forceinline__ int bwd_swizzle(int row) {
  static_assert(RB == 128 || RB == 256, "rows of 64 or 128 two-byte elements");
  constexpr int RPB = 256 / RB, Q = RB / 64, CK = RB / 16;
  const int h = row / RPB;
  return ((h % Q) * 4 + (h / Q) % 4) % CK;
}

template <int DH, int DV>
struct BwdDmaCfg {
  static constexpr int QRB = DH * 2, ZRB = DV * 2;          // row bytes
  static constexpr int QT = 64 * QRB, ZT = 64 * ZRB;        // tile bytes
  static constexpr int AUX = 2048;                          // L (1 KB), D (1 KB)
  static constexpr int STAGE = QT + ZT + AUX, NS = 3;
  static constexpr int Q_WIN = QT / 1024 / 4, Z_WIN = ZT / 1024 / 4;   // per wave
  static constexpr int LDS = NS * STAGE;
};

template <typename T, int DH, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BwdCfg<DH, DV>::KV_OCC, 2)))
void attn_bwd_kv_dma_kernel(AttnBwdParams p) {
  typedef BwdCfg<DH, DV> C;
  typedef BwdDmaCfg<DH, DV> D;
  typedef typename Elem<T>::vec vec;
  typedef typename Elem<T>::vec4 vec4;
  __shared__ __attribute__((aligned(1024))) char smem[D::LDS];
  const unsigned lds_base = (unsigned)(size_t)(__attribute__((address_space(3))) char*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int BH = p.B * p.h;
  const int kt = blockIdx.x / BH;             // key tile (earliest keys first: most queries)
  const int bh = blockIdx.x - kt * BH;
  const int b = bh / p.h, r = bh - b * p.h;
  const int k0 = kt * 128, k0w = k0 + 32 * wave;
  const int key = k0w + l32;                  // this lane's key
  int kvalid = p.n_k;
  if (p.key_len) kvalid = min(kvalid, p.key_len[b]);

  const T* Qb = reinterpret_cast<const T*>(p.Q) + (size_t)bh * p.n_q * DH;
  const T* Kb = reinterpret_cast<const T*>(p.K) + (size_t)bh * p.n_k * DH;
  const T* Vb = reinterpret_cast<const T*>(p.V) + (size_t)bh * p.n_k * DV;
  const T* Zb = reinterpret_cast<const T*>(p.dZ) + (size_t)b * p.n_q * p.ldz + (size_t)r * DV;
  // causal / key-padding masks only (the host launches this kernel without a
  // boolean mask or additive bias)
  const float* lse = p.lse2 + (size_t)bh * p.n_q;
  const float* dsm = p.dsum + (size_t)bh * p.n_q;

  vec kf[C::KCH], vf[C::VCH];
  #pragma unroll
  for (int c = 0; c < C::KCH; ++c)
    kf[c] = key < p.n_k ? *reinterpret_cast<const vec*>(Kb + (size_t)key * DH + 16 * c + 8 * g)
                        : zero_vec<vec>();
  #pragma unroll
  for (int c = 0; c < C::VCH; ++c)
    vf[c] = key < p.n_k ? *reinterpret_cast<const vec*>(Vb + (size_t)key * DV + 16 * c + 8 * g)
                        : zero_vec<vec>();
  // the loop's waits count only the direct loads: the compiler's wait for
  // these rows is taken here, once, not before every product in the loop
  // (where a full vmcnt wait would also drain the tiles loaded ahead)
  #pragma unroll
  for (int c = 0; c < C::KCH; ++c) asm volatile("" : "+v"(kf[c]));
  #pragma unroll
  for (int c = 0; c < C::VCH; ++c) asm volatile("" : "+v"(vf[c]));

  floatx16 dk[C::NDH], dv[C::NDV];
  #pragma unroll
  for (int d = 0; d < C::NDH; ++d)
    #pragma unroll
    for (int i = 0; i < 16; ++i) dk[d][i] = 0.f;
  #pragma unroll
  for (int d = 0; d < C::NDV; ++d)
    #pragma unroll
    for (int i = 0; i < 16; ++i) dv[d][i] = 0.f;

  const int qb0 = (p.causal ? k0 : 0) / C::BR;
  const int nqb = (k0 < kvalid) ? (p.n_q + C::BR - 1) / C::BR : qb0;

  // ---- direct loads: window q of this wave covers tile bytes
  // (wave * WIN + q) KB; lane i fills 16 bytes at 16 i, i.e. tile row t / RB,
  // slot (t % RB) / 16, from the global chunk the slot holds.  Rows past n_q
  // read the last row (never used: their weights are 0).
  auto q_row = [&](int win) { return (win * 1024 + 16 * lane) / D::QRB; };
  auto z_row = [&](int win) { return (win * 1024 + 16 * lane) / D::ZRB; };
  auto q_chunk = [&](int win) {
    const int t = win * 1024 + 16 * lane, row = t / D::QRB;
    return ((t % D::QRB) / 16) ^ bwd_swizzle<D::QRB>(row);
  };
  auto z_chunk = [&](int win) {
    const int t = win * 1024 + 16 * lane, row = t / D::ZRB;
    return ((t % D::ZRB) / 16) ^ bwd_swizzle<D::ZRB>(row);
  };
  // L (wave 0) and D (wave 1): lane i loads rows 4 (i % 16) .. +3 of the
  // tile; lanes 16..63 repeat them into spare LDS bytes.  n_q % 4 == 0, so
  // a 4-row chunk is either all valid or all past n_q (then the last chunk).
  const bool aux_wave = wave < 2;
  const float* aux_src = wave == 0 ? lse : dsm;
  auto issue = [&](int qb) {
    const int q0 = qb * C::BR;
    const unsigned st = lds_base + (unsigned)((qb % D::NS) * D::STAGE);
    const char* qg = reinterpret_cast<const char*>(Qb + (size_t)q0 * DH);
    const char* zg = reinterpret_cast<const char*>(Zb + (size_t)q0 * p.ldz);
    const int last = p.n_q - 1 - q0;   // last valid row of the tile
    #pragma unroll
    for (int q = 0; q < D::Q_WIN; ++q) {
      const int win = wave * D::Q_WIN + q;
      const unsigned off = (unsigned)(min(q_row(win), last) * D::QRB + q_chunk(win) * 16);
      lds_dma16(qg, off, st + win * 1024);
    }
    #pragma unroll
    for (int q = 0; q < D::Z_WIN; ++q) {
      const int win = wave * D::Z_WIN + q;
      const unsigned off =
          (unsigned)(min(z_row(win), last) * p.ldz * 2 + z_chunk(win) * 16);
      lds_dma16(zg, off, st + D::QT + win * 1024);
    }
    if (aux_wave) {
      const int row = min(q0 + 4 * (lane & 15), p.n_q - 4);
      lds_dma16(aux_src, (unsigned)row * 4u, st + D::QT + D::ZT + wave * 1024);
    }
  };

  // ---- per-lane LDS read offsets within a stage (bytes) ----------------------
  // 16-byte row reads: row 32 sb + l32, chunk 2 c + g (the swizzle depends on
  // the row through l32 only).  Transposing reads: row 32 sb + 16 st + 8 hh +
  // 4 g + (lane % 16) / 4, columns 32 d + scol; the swizzle depends on the row
  // through 8 hh + 4 g + (lane % 16) / 4, so hh gets its own base.
  int qro[C::KCH], zro[C::VCH], qtr[C::NDH][2], ztr[C::NDV][2];
  #pragma unroll
  for (int c = 0; c < C::KCH; ++c)
    qro[c] = l32 * D::QRB + (((2 * c + g) ^ bwd_swizzle<D::QRB>(l32)) * 16);
  #pragma unroll
  for (int c = 0; c < C::VCH; ++c)
    zro[c] = D::QT + l32 * D::ZRB + (((2 * c + g) ^ bwd_swizzle<D::ZRB>(l32)) * 16);
  {
    const int scol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    #pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int vr = 8 * hh + 4 * g + ((lane & 15) >> 2);
      #pragma unroll
      for (int d = 0; d < C::NDH; ++d) {
        const int col = d * 32 + scol;
        qtr[d][hh] = vr * D::QRB + (((col / 8) ^ bwd_swizzle<D::QRB>(vr)) * 16) + (col % 8) * 2;
      }
      #pragma unroll
      for (int d = 0; d < C::NDV; ++d) {
        const int col = d * 32 + scol;
        ztr[d][hh] = D::QT + vr * D::ZRB + (((col / 8) ^ bwd_swizzle<D::ZRB>(vr)) * 16) +
                     (col % 8) * 2;
      }
    }
  }
  const int aro = D::QT + D::ZT + 16 * g;   // L of query 4 g + 8 a + 32 sb: + 4 (8 a + 32 sb)

  constexpr int LOADS = D::Q_WIN + D::Z_WIN;   // per wave per tile, plus one on waves 0, 1
  if (nqb > qb0) issue(qb0);
  if (nqb > qb0 + 1) issue(qb0 + 1);
  const float cs = p.scale_log2;

  for (int qb = qb0; qb < nqb; ++qb) {
    // tile qb has landed once only tile qb+1's loads are outstanding; after
    // the barrier no wave reads tile qb-1, whose stage gets tile qb+2
    if (qb + 1 < nqb) {
      if (aux_wave) wait_vm_lds<LOADS + 1>();
      else wait_vm_lds<LOADS>();
    } else {
      wait_vm_lds<0>();
    }
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    if (qb + 2 < nqb) issue(qb + 2);

    unsigned st_addr = lds_base + (unsigned)((qb % D::NS) * D::STAGE);
    asm("" : "+s"(st_addr));
    unsigned qa_addr[C::KCH], za_addr[C::VCH], qt_addr[C::NDH][2], zt_addr[C::NDV][2], a_addr;
    #pragma unroll
    for (int c = 0; c < C::KCH; ++c) {
      qa_addr[c] = st_addr + (unsigned)qro[c];
      asm("" : "+v"(qa_addr[c]));
    }
    #pragma unroll
    for (int c = 0; c < C::VCH; ++c) {
      za_addr[c] = st_addr + (unsigned)zro[c];
      asm("" : "+v"(za_addr[c]));
    }
    #pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      #pragma unroll
      for (int d = 0; d < C::NDH; ++d) {
        qt_addr[d][hh] = st_addr + (unsigned)qtr[d][hh];
        asm("" : "+v"(qt_addr[d][hh]));
      }
      #pragma unroll
      for (int d = 0; d < C::NDV; ++d) {
        zt_addr[d][hh] = st_addr + (unsigned)ztr[d][hh];
        asm("" : "+v"(zt_addr[d][hh]));
      }
    }
    a_addr = st_addr + (unsigned)aro;
    asm("" : "+v"(a_addr));

    const int q0 = qb * C::BR;
    #pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int qs0 = q0 + 32 * sb;
      if ((p.causal && qs0 + 31 < k0w) || k0w >= kvalid || qs0 >= p.n_q) continue;
      floatx16 sacc, dpacc;
      #pragma unroll
      for (int i = 0; i < 16; ++i) {
        sacc[i] = 0.f;
        dpacc[i] = 0.f;
      }
      // every operand of the two products read first (their LDS latencies
      // overlap), then the products
      vec qop[C::KCH], zop[C::VCH];
      #pragma unroll
      for (int c = 0; c < C::KCH; ++c) qop[c] = lds_load_at<vec>(qa_addr[c] + 32 * sb * D::QRB);
      #pragma unroll
      for (int c = 0; c < C::VCH; ++c) zop[c] = lds_load_at<vec>(za_addr[c] + 32 * sb * D::ZRB);
      #pragma unroll
      for (int c = 0; c < C::KCH; ++c) mfma_chunk(sacc, qop[c], kf[c]);
      #pragma unroll
      for (int c = 0; c < C::VCH; ++c) mfma_chunk(dpacc, zop[c], vf[c]);
      __builtin_amdgcn_sched_group_barrier(0x100, C::KCH + C::VCH, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, C::KCH + C::VCH, 0);
      // L and D of slot i's query 32 sb + 8 (i/4) + 4 g + i%4
      floatx4 lq[4], dq[4];
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        lq[a] = lds_load_at<floatx4>(a_addr + 4 * (8 * a + 32 * sb));
        dq[a] = lds_load_at<floatx4>(a_addr + 1024 + 4 * (8 * a + 32 * sb));
      }
      const bool need_mask = (p.causal && qs0 < k0w + 31) || (k0w + 31 >= kvalid) ||
                             (qs0 + 31 >= p.n_q);
      // a forbidden score's exponent becomes -inf (weight exactly 0), without
      // a branch per score; the test runs on boundary tiles only
      if (need_mask) {
        #pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = qs0 + 8 * (i >> 2) + 4 * g + (i & 3);
          const float x = fmaf(sacc[i], cs, -lq[i >> 2][i & 3]);
          sacc[i] = bwd_allowed(p, nullptr, q, key, kvalid) ? x : -INFINITY;
        }
      } else {
        #pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = fmaf(sacc[i], cs, -lq[i >> 2][i & 3]);
      }
      #pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float a = __builtin_amdgcn_exp2f(sacc[i]);
        sacc[i] = a;
        dpacc[i] = a * (dpacc[i] - dq[i >> 2][i & 3]);
      }
      #pragma unroll
      for (int st = 0; st < 2; ++st) {
        floatx8 af, sf;
        #pragma unroll
        for (int t = 0; t < 8; ++t) {
          af[t] = sacc[8 * st + t];
          sf[t] = dpacc[8 * st + t];
        }
        const vec ab = Cvt<T>::eight(af);
        const vec sbv = Cvt<T>::eight(sf);
        #pragma unroll
        for (int d = 0; d < C::NDV; ++d) {
          const unsigned o = (32 * sb + 16 * st) * D::ZRB;
          const vec4 lo = lds_read_tr4_at<T>(zt_addr[d][0] + o);
          const vec4 hi = lds_read_tr4_at<T>(zt_addr[d][1] + o);
          const vec za = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          mfma_chunk(dv[d], za, ab);
        }
        #pragma unroll
        for (int d = 0; d < C::NDH; ++d) {
          const unsigned o = (32 * sb + 16 * st) * D::QRB;
          const vec4 lo = lds_read_tr4_at<T>(qt_addr[d][0] + o);
          const vec4 hi = lds_read_tr4_at<T>(qt_addr[d][1] + o);
          const vec qa = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          mfma_chunk(dk[d], qa, sbv);
        }
      }
    }
  }

  if (key < p.n_k) {
    const size_t krow = p.grad_concat ? ((size_t)b * p.n_k + key) * p.h + r
                                      : (size_t)bh * p.n_k + key;
    const size_t kro = krow * DH;
    const size_t vro = krow * DV;
    #pragma unroll
    for (int d = 0; d < C::NDH; ++d)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int e0 = d * 32 + 8 * a + 4 * g;
        store4(p.dK, p.g_dtype, kro + e0, p.vec_dk, DH - e0, dk[d][4 * a] * p.scale,
               dk[d][4 * a + 1] * p.scale, dk[d][4 * a + 2] * p.scale, dk[d][4 * a + 3] * p.scale);
      }
    #pragma unroll
    for (int d = 0; d < C::NDV; ++d)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int e0 = d * 32 + 8 * a + 4 * g;
        store4(p.dV, p.g_dtype, vro + e0, p.vec_dv, DV - e0, dv[d][4 * a], dv[d][4 * a + 1],
               dv[d][4 * a + 2], dv[d][4 * a + 3]);
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (128 queries, b*h + r); a wave owns 32 queries.
// ---------------------------------------------------------------------------
template <typename T, int DH, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_q_kernel(AttnBwdParams p) {
  typedef BwdCfg<DH, DV> C;
  typedef typename Elem<T>::vec vec;
  typedef typename Elem<T>::vec4 vec4;
  __shared__ __attribute__((aligned(16))) T Ks[2][C::HTILE];
  __shared__ __attribute__((aligned(16))) T Vs[2][C::VTILE];
  constexpr int tdt = __is_same(T, bf16) ? kBF16 : kF16;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int BH = p.B * p.h;
  const int nqt = (p.n_q + 127) / 128;
  const int qt_rank = blockIdx.x / BH;
  const int bh = blockIdx.x - qt_rank * BH;
  const int qt = p.causal ? (nqt - 1 - qt_rank) : qt_rank;   // causal: most keys first
  const int b = bh / p.h, r = bh - b * p.h;
  const int q0 = qt * 128, q0w = q0 + 32 * wave;
  const int qi = q0w + l32;                    // this lane's query
  int kvalid = p.n_k;
  if (p.key_len) kvalid = min(kvalid, p.key_len[b]);
  int kend = kvalid;
  if (p.causal) kend = min(kend, q0 + 128);
  const int nkb = kend > 0 ? (kend + C::BR - 1) / C::BR : 0;

  const T* Qb = reinterpret_cast<const T*>(p.Q) + (size_t)bh * p.n_q * p.d_h;
  const T* Kb = reinterpret_cast<const T*>(p.K) + (size_t)bh * p.n_k * p.d_h;
  const T* Vb = reinterpret_cast<const T*>(p.V) + (size_t)bh * p.n_k * p.d_vh;
  const size_t zrow = ((size_t)b * p.n_q + qi) * p.ldz + (size_t)r * p.d_vh;
  const uint8_t* G = p.allowed ? p.allowed + (size_t)b * p.allowed_batch_stride : nullptr;
  const float* M = p.add ? p.add + (size_t)b * p.add_batch_stride : nullptr;

  // this lane's query row of Q and dZ as B operands
  vec qf[C::KCH], zf[C::VCH];
  #pragma unroll
  for (int c = 0; c < C::KCH; ++c)
    qf[c] = qi < p.n_q ? load_chunk<T>(Qb + (size_t)qi * p.d_h, 16 * c + 8 * g, p.d_h, p.vec_q)
                       : zero_vec<vec>();
  #pragma unroll
  for (int c = 0; c < C::VCH; ++c)
    zf[c] = qi < p.n_q ? load8_as<T>(p.dZ, p.z_dtype, zrow, 16 * c + 8 * g, p.d_vh, p.vec_z)
                       : zero_vec<vec>();
  const float Lq = qi < p.n_q ? p.lse2[(size_t)bh * p.n_q + qi] : INFINITY;
  const float Dq = qi < p.n_q ? p.dsum[(size_t)bh * p.n_q + qi] : 0.f;

  floatx16 dq[C::NDH];
  #pragma unroll
  for (int d = 0; d < C::NDH; ++d)
    #pragma unroll
    for (int i = 0; i < 16; ++i) dq[d][i] = 0.f;

  TileStager<T, DH, C::HROW, C::H_PER_T, C::NT> kst;
  TileStager<T, DV, C::VROW, C::V_PER_T, C::NT> vst;
  auto load_tile = [&](int kb) {
    const int kk0 = kb * C::BR;
    kst.load(Kb, tdt, 0, p.d_h, kk0, p.n_k, p.d_h, p.vec_k, tid);
    vst.load(Vb, tdt, 0, p.d_vh, kk0, p.n_k, p.d_vh, p.vec_v, tid);
  };
  auto store_tile = [&](int buf) {
    kst.store(Ks[buf], tid);
    vst.store(Vs[buf], tid);
  };
  if (nkb > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  if (nkb > 1) load_tile(1);

  const int srow = 4 * g + ((lane & 15) >> 2);
  const int scol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const float cs = p.scale_log2;

  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    const T* ks = Ks[cur];
    const T* vs = Vs[cur];
    const int kk0 = kb * C::BR;
    #pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int ks0 = kk0 + 32 * sb;
      if ((p.causal && ks0 > q0w + 31) || ks0 >= kvalid || q0w >= p.n_q) continue;
      floatx16 sacc, dpacc;
      #pragma unroll
      for (int i = 0; i < 16; ++i) {
        sacc[i] = 0.f;
        dpacc[i] = 0.f;
      }
      // S^T = K Q^T (lane: query l32; registers: keys), dA^T = V dZ^T
      #pragma unroll
      for (int c = 0; c < C::KCH; ++c) {
        const vec ka = *reinterpret_cast<const vec*>(&ks[(32 * sb + l32) * C::HROW + 16 * c + 8 * g]);
        mfma_chunk(sacc, ka, qf[c]);
      }
      #pragma unroll
      for (int c = 0; c < C::VCH; ++c) {
        const vec va = *reinterpret_cast<const vec*>(&vs[(32 * sb + l32) * C::VROW + 16 * c + 8 * g]);
        mfma_chunk(dpacc, va, zf[c]);
      }
      const bool need_mask = (p.causal && ks0 + 31 > q0w) || (ks0 + 31 >= kvalid) ||
                             (q0w + 31 >= p.n_q) || G != nullptr || M != nullptr;
      // forbidden scores: exponent -inf (weight exactly 0), no branch per score
      if (need_mask) {
        #pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = ks0 + 8 * (i >> 2) + 4 * g + (i & 3);
          const bool ok = bwd_allowed(p, G, qi, key, kvalid);
          float x;
          if (M != nullptr) {
            x = sacc[i] * cs;
            if (ok) x = fmaf(M[(size_t)qi * p.n_k + key], kLog2e, x);
            x -= Lq;
          } else {
            x = fmaf(sacc[i], cs, -Lq);
          }
          sacc[i] = ok ? x : -INFINITY;
        }
      } else {
        #pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = fmaf(sacc[i], cs, -Lq);
      }
      #pragma unroll
      for (int i = 0; i < 16; ++i)
        sacc[i] = __builtin_amdgcn_exp2f(sacc[i]) * (dpacc[i] - Dq);   // dS^T

      // dQ^T += K^T dS^T (slot permutation as in the forward's value product)
      #pragma unroll
      for (int st = 0; st < 2; ++st) {
        floatx8 sf;
        #pragma unroll
        for (int t = 0; t < 8; ++t) sf[t] = sacc[8 * st + t];
        const vec sbv = Cvt<T>::eight(sf);
        #pragma unroll
        for (int d = 0; d < C::NDH; ++d) {
          const T* k0p = &ks[(32 * sb + 16 * st + srow) * C::HROW + d * 32 + scol];
          const vec4 lo = lds_read_tr4<T>(k0p);
          const vec4 hi = lds_read_tr4<T>(k0p + 8 * C::HROW);
          const vec ka = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          mfma_chunk(dq[d], ka, sbv);
        }
      }
    }
    if (kb + 1 < nkb) store_tile(cur ^ 1);
    __syncthreads();
    if (kb + 2 < nkb) load_tile(kb + 2);
  }

  if (qi < p.n_q) {
    const size_t qro = (p.grad_concat ? ((size_t)b * p.n_q + qi) * p.h + r
                                      : (size_t)bh * p.n_q + qi) * p.d_h;
    #pragma unroll
    for (int d = 0; d < C::NDH; ++d)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int e0 = d * 32 + 8 * a + 4 * g;
        store4(p.dQ, p.g_dtype, qro + e0, p.vec_dq, p.d_h - e0, dq[d][4 * a] * p.scale,
               dq[d][4 * a + 1] * p.scale, dq[d][4 * a + 2] * p.scale, dq[d][4 * a + 3] * p.scale);
      }
  }
}

// ---------------------------------------------------------------------------
// dQ with direct-to-LDS key tiles (2-byte K and V of exactly DH / DV columns,
// 16-byte aligned rows): same products, summation order and results as
// attn_bwd_q_kernel, with the 64-row K and V tiles moving from global memory
// straight into LDS (three stages in flight).  K is read with both patterns
// (16-byte rows for S^T = K Q^T, transposing reads for dQ^T += K^T dS^T), V
// with row reads only; both use the permutation bwd_swizzle.
// ---------------------------------------------------------------------------
template <int DH, int DV>
struct BwdQDmaCfg {
  // waves per SIMD: three for heads of 64 (measured 3 % faster than two;
  // 140 VGPRs, 48 KB of LDS per workgroup), else two
  static constexpr int OCC = (DH + DV <= 128) ? 3 : 2;
  static constexpr int KRB = DH * 2, VRB = DV * 2;
  static constexpr int KT = 64 * KRB, VT = 64 * VRB;
  static constexpr int STAGE = KT + VT, NS = 3;
  static constexpr int K_WIN = KT / 1024 / 4, V_WIN = VT / 1024 / 4;
  static constexpr int LDS = NS * STAGE;
};

template <typename T, int DH, int DV>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(BwdQDmaCfg<DH, DV>::OCC, BwdQDmaCfg<DH, DV>::OCC)))
void attn_bwd_q_dma_kernel(AttnBwdParams p) {
  typedef BwdCfg<DH, DV> C;
  typedef BwdQDmaCfg<DH, DV> D;
  typedef typename Elem<T>::vec vec;
  typedef typename Elem<T>::vec4 vec4;
  __shared__ __attribute__((aligned(1024))) char smem[D::LDS];
  const unsigned lds_base = (unsigned)(size_t)(__attribute__((address_space(3))) char*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int BH = p.B * p.h;
  const int nqt = (p.n_q + 127) / 128;
  const int qt_rank = blockIdx.x / BH;
  const int bh = blockIdx.x - qt_rank * BH;
  const int qt = p.causal ? (nqt - 1 - qt_rank) : qt_rank;   // causal: most keys first
  const int b = bh / p.h, r = bh - b * p.h;
  const int q0 = qt * 128, q0w = q0 + 32 * wave;
  const int qi = q0w + l32;                    // this lane's query
  int kvalid = p.n_k;
  if (p.key_len) kvalid = min(kvalid, p.key_len[b]);
  int kend = kvalid;
  if (p.causal) kend = min(kend, q0 + 128);
  const int nkb = kend > 0 ? (kend + C::BR - 1) / C::BR : 0;

  const T* Qb = reinterpret_cast<const T*>(p.Q) + (size_t)bh * p.n_q * DH;
  const T* Kb = reinterpret_cast<const T*>(p.K) + (size_t)bh * p.n_k * DH;
  const T* Vb = reinterpret_cast<const T*>(p.V) + (size_t)bh * p.n_k * DV;
  const size_t zrow = ((size_t)b * p.n_q + qi) * p.ldz + (size_t)r * DV;

  vec qf[C::KCH], zf[C::VCH];
  #pragma unroll
  for (int c = 0; c < C::KCH; ++c)
    qf[c] = qi < p.n_q ? *reinterpret_cast<const vec*>(Qb + (size_t)qi * DH + 16 * c + 8 * g)
                       : zero_vec<vec>();
  #pragma unroll
  for (int c = 0; c < C::VCH; ++c)
    zf[c] = qi < p.n_q ? load8_as<T>(p.dZ, p.z_dtype, zrow, 16 * c + 8 * g, DV, p.vec_z)
                       : zero_vec<vec>();
  const float Lq0 = qi < p.n_q ? p.lse2[(size_t)bh * p.n_q + qi] : INFINITY;
  const float Dq0 = qi < p.n_q ? p.dsum[(size_t)bh * p.n_q + qi] : 0.f;
  // waited for here, once (see the dK/dV kernel)
  #pragma unroll
  for (int c = 0; c < C::KCH; ++c) asm volatile("" : "+v"(qf[c]));
  #pragma unroll
  for (int c = 0; c < C::VCH; ++c) asm volatile("" : "+v"(zf[c]));
  float Lq = Lq0, Dq = Dq0;
  asm volatile("" : "+v"(Lq), "+v"(Dq));

  floatx16 dq[C::NDH];
  #pragma unroll
  for (int d = 0; d < C::NDH; ++d)
    #pragma unroll
    for (int i = 0; i < 16; ++i) dq[d][i] = 0.f;

  // direct loads (window mapping as in attn_bwd_kv_dma_kernel); rows past
  // n_k read the last key (masked: weight 0)
  auto k_row = [&](int win) { return (win * 1024 + 16 * lane) / D::KRB; };
  auto v_row = [&](int win) { return (win * 1024 + 16 * lane) / D::VRB; };
  auto k_chunk = [&](int win) {
    const int t = win * 1024 + 16 * lane, row = t / D::KRB;
    return ((t % D::KRB) / 16) ^ bwd_swizzle<D::KRB>(row);
  };
  auto v_chunk = [&](int win) {
    const int t = win * 1024 + 16 * lane, row = t / D::VRB;
    return ((t % D::VRB) / 16) ^ bwd_swizzle<D::VRB>(row);
  };
  auto issue = [&](int kb) {
    const int kk0 = kb * C::BR;
    const unsigned st = lds_base + (unsigned)((kb % D::NS) * D::STAGE);
    const char* kg = reinterpret_cast<const char*>(Kb + (size_t)kk0 * DH);
    const char* vg = reinterpret_cast<const char*>(Vb + (size_t)kk0 * DV);
    const int last = p.n_k - 1 - kk0;
    #pragma unroll
    for (int q = 0; q < D::K_WIN; ++q) {
      const int win = wave * D::K_WIN + q;
      lds_dma16(kg, (unsigned)(min(k_row(win), last) * D::KRB + k_chunk(win) * 16),
                st + win * 1024);
    }
    #pragma unroll
    for (int q = 0; q < D::V_WIN; ++q) {
      const int win = wave * D::V_WIN + q;
      lds_dma16(vg, (unsigned)(min(v_row(win), last) * D::VRB + v_chunk(win) * 16),
                st + D::KT + win * 1024);
    }
  };

  int kro[C::KCH], vro[C::VCH], ktr[C::NDH][2];
  #pragma unroll
  for (int c = 0; c < C::KCH; ++c)
    kro[c] = l32 * D::KRB + (((2 * c + g) ^ bwd_swizzle<D::KRB>(l32)) * 16);
  #pragma unroll
  for (int c = 0; c < C::VCH; ++c)
    vro[c] = D::KT + l32 * D::VRB + (((2 * c + g) ^ bwd_swizzle<D::VRB>(l32)) * 16);
  {
    const int scol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    #pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int vr = 8 * hh + 4 * g + ((lane & 15) >> 2);
      #pragma unroll
      for (int d = 0; d < C::NDH; ++d) {
        const int col = d * 32 + scol;
        ktr[d][hh] = vr * D::KRB + (((col / 8) ^ bwd_swizzle<D::KRB>(vr)) * 16) + (col % 8) * 2;
      }
    }
  }

  constexpr int LOADS = D::K_WIN + D::V_WIN;
  if (nkb > 0) issue(0);
  if (nkb > 1) issue(1);
  const float cs = p.scale_log2;

  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) wait_vm_lds<LOADS>();
    else wait_vm_lds<0>();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    if (kb + 2 < nkb) issue(kb + 2);

    unsigned st_addr = lds_base + (unsigned)((kb % D::NS) * D::STAGE);
    asm("" : "+s"(st_addr));
    unsigned ka_addr[C::KCH], va_addr[C::VCH], kt_addr[C::NDH][2];
    #pragma unroll
    for (int c = 0; c < C::KCH; ++c) {
      ka_addr[c] = st_addr + (unsigned)kro[c];
      asm("" : "+v"(ka_addr[c]));
    }
    #pragma unroll
    for (int c = 0; c < C::VCH; ++c) {
      va_addr[c] = st_addr + (unsigned)vro[c];
      asm("" : "+v"(va_addr[c]));
    }
    #pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      #pragma unroll
      for (int d = 0; d < C::NDH; ++d) {
        kt_addr[d][hh] = st_addr + (unsigned)ktr[d][hh];
        asm("" : "+v"(kt_addr[d][hh]));
      }

    const int kk0 = kb * C::BR;
    #pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int ks0 = kk0 + 32 * sb;
      if ((p.causal && ks0 > q0w + 31) || ks0 >= kvalid || q0w >= p.n_q) continue;
      floatx16 sacc, dpacc;
      #pragma unroll
      for (int i = 0; i < 16; ++i) {
        sacc[i] = 0.f;
        dpacc[i] = 0.f;
      }
      // operands read first, then the products (as in the dK/dV pass)
      vec kop[C::KCH], vop[C::VCH];
      #pragma unroll
      for (int c = 0; c < C::KCH; ++c) kop[c] = lds_load_at<vec>(ka_addr[c] + 32 * sb * D::KRB);
      #pragma unroll
      for (int c = 0; c < C::VCH; ++c) vop[c] = lds_load_at<vec>(va_addr[c] + 32 * sb * D::VRB);
      #pragma unroll
      for (int c = 0; c < C::KCH; ++c) mfma_chunk(sacc, kop[c], qf[c]);
      #pragma unroll
      for (int c = 0; c < C::VCH; ++c) mfma_chunk(dpacc, vop[c], zf[c]);
      __builtin_amdgcn_sched_group_barrier(0x100, C::KCH + C::VCH, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, C::KCH + C::VCH, 0);
      const bool need_mask = (p.causal && ks0 + 31 > q0w) || (ks0 + 31 >= kvalid) ||
                             (q0w + 31 >= p.n_q);
      // forbidden scores: exponent -inf (weight exactly 0), boundary tiles only
      if (need_mask) {
        #pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = ks0 + 8 * (i >> 2) + 4 * g + (i & 3);
          const float x = fmaf(sacc[i], cs, -Lq);
          sacc[i] = bwd_allowed(p, nullptr, qi, key, kvalid) ? x : -INFINITY;
        }
      } else {
        #pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = fmaf(sacc[i], cs, -Lq);
      }
      #pragma unroll
      for (int i = 0; i < 16; ++i)
        sacc[i] = __builtin_amdgcn_exp2f(sacc[i]) * (dpacc[i] - Dq);   // dS^T

      #pragma unroll
      for (int st = 0; st < 2; ++st) {
        floatx8 sf;
        #pragma unroll
        for (int t = 0; t < 8; ++t) sf[t] = sacc[8 * st + t];
        const vec sbv = Cvt<T>::eight(sf);
        #pragma unroll
        for (int d = 0; d < C::NDH; ++d) {
          const unsigned o = (32 * sb + 16 * st) * D::KRB;
          const vec4 lo = lds_read_tr4_at<T>(kt_addr[d][0] + o);
          const vec4 hi = lds_read_tr4_at<T>(kt_addr[d][1] + o);
          const vec ka = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          mfma_chunk(dq[d], ka, sbv);
        }
      }
    }
  }

  if (qi < p.n_q) {
    const size_t qro = (p.grad_concat ? ((size_t)b * p.n_q + qi) * p.h + r
                                      : (size_t)bh * p.n_q + qi) * DH;
    #pragma unroll
    for (int d = 0; d < C::NDH; ++d)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int e0 = d * 32 + 8 * a + 4 * g;
        store4(p.dQ, p.g_dtype, qro + e0, p.vec_dq, DH - e0, dq[d][4 * a] * p.scale,
               dq[d][4 * a + 1] * p.scale, dq[d][4 * a + 2] * p.scale, dq[d][4 * a + 3] * p.scale);
      }
  }
}

}  // namespace mha
