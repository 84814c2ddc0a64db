// General GEMM for the gradients of the projections (gfx950):
// C[M, N] = A[M, K] * W[K, N] with fp32 accumulation, where either operand
// may be stored transposed and each operand has its own element type.
//
// The gradients of the layer's products (calculus on page "Multi-head
// attention and self-attention", Definition: Y = Z W^O, Q_r = X W_r^Q, ...)
// are products with one transposed factor: dZ = dY (W^O)^T, dW^O = Z^T dY,
// dW^Q = X^T dQ, dX = dQ (W^Q)^T.  This kernel takes them all:
//   A: a_trans = 0 -> A(m, k) = A[m * lda + k];  1 -> A(m, k) = A[k * lda + m]
//   W: w_trans = 0 -> W(k, n) = W[k * ldw + n];  1 -> W(k, n) = W[n * ldw + k]
// Operands of any of the three element types are rounded to the compute type
// T (nearest even) as they are staged; C is written in its own type.
//
// Design (ours): 128 x 128 workgroup tile, four waves of 64 x 64, C^T = W^T A^T
// with 32x32 MFMAs as in gemm_kernel.  Both LDS tiles are k-contiguous rows
// (A tile [m][k], W tile [n][k]); an operand whose memory is contiguous along
// k is copied in 16-byte chunks, the other is loaded along m (or n) and
// scattered into the rows.  Register staging, one LDS buffer.
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace mha {

// VEC consecutive elements (of `count` valid ones) at element `idx` of an
// array of type `dt`, rounded to T; `vec_ok`: a full chunk may be read with
// vector loads.
template <typename T>
__device__ __forceinline__ typename Elem<T>::vec load_vec_as(const void* base, int dt, size_t idx,
                                                             int count, bool vec_ok) {
  typedef typename Elem<T>::vec V;
  constexpr int VEC = Elem<T>::VEC;
  V v;
  if (vec_ok && count >= VEC) {
    if (dt == kF32) {
      const float* p = reinterpret_cast<const float*>(base) + idx;
      #pragma unroll
      for (int q = 0; q < VEC / 4; ++q) {
        const floatx4 f = *reinterpret_cast<const floatx4*>(p + 4 * q);
        #pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * q + e] = (T)f[e];
      }
    } else if (dt == kBF16) {
      const bf16* p = reinterpret_cast<const bf16*>(base) + idx;
      #pragma unroll
      for (int q = 0; q < VEC / 4; ++q) {
        const bf16x4 f = *reinterpret_cast<const bf16x4*>(p + 4 * q);
        #pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * q + e] = (T)(float)f[e];
      }
    } else {
      const f16* p = reinterpret_cast<const f16*>(base) + idx;
      #pragma unroll
      for (int q = 0; q < VEC / 4; ++q) {
        const f16x4 f = *reinterpret_cast<const f16x4*>(p + 4 * q);
        #pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * q + e] = (T)(float)f[e];
      }
    }
    return v;
  }
  #pragma unroll
  for (int e = 0; e < VEC; ++e) {
    float x = 0.f;
    if (e < count) {
      if (dt == kF32) x = reinterpret_cast<const float*>(base)[idx + e];
      else if (dt == kBF16) x = (float)reinterpret_cast<const bf16*>(base)[idx + e];
      else x = (float)reinterpret_cast<const f16*>(base)[idx + e];
    }
    v[e] = (T)x;
  }
  return v;
}

template <typename T>
__global__ __launch_bounds__(256) void gemm_any_kernel(GemmAny P) {
  typedef Elem<T> E;
  typedef typename E::vec vec;
  constexpr int VEC = E::VEC;
  constexpr int BM = 128, BN = 128, WM = 64, WN = 64, NT = 256, KCH = 2;
  constexpr int BK = KCH * 2 * VEC;          // 32 (2-byte) / 16 (fp32)
  constexpr int PAD = BK + VEC;              // LDS row stride (elements)
  constexpr int CH = BM * BK / VEC;          // chunks per tile (A and W alike)
  constexpr int PER_T = CH / NT;
  static_assert(CH % NT == 0, "tile/thread mismatch");
  __shared__ __attribute__((aligned(16))) T Xs[BM * PAD];
  __shared__ __attribute__((aligned(16))) T Wt[BN * PAD];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = (P.N + BN - 1) / BN;
  const int tiles = ((P.M + BM - 1) / BM) * tiles_n;
  const int ks = blockIdx.x / tiles;                  // K partition (split-K)
  const int tile = blockIdx.x - ks * tiles;
  const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = P.M, N = P.N;
  // this workgroup's K range [kb, K): loads index k from kb, bounded by K
  const int kb = ks * P.kchunk;
  const int K = min(P.K, kb + P.kchunk);

  floatx16 acc[2][2];
  #pragma unroll
  for (int j = 0; j < 2; ++j)
    #pragma unroll
    for (int i = 0; i < 2; ++i)
      #pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.f;

  vec xr[PER_T], wr[PER_T];
  // chunk ci of a tile: k-contiguous layout -> (row ci / (BK/VEC), k chunk);
  // row-contiguous layout -> (k row ci / (128/VEC), row chunk)
  auto load_stage = [&](int k0) {
    #pragma unroll
    for (int t = 0; t < PER_T; ++t) {
      const int ci = tid + t * NT;
      if (!P.a_trans) {
        const int row = ci / (BK / VEC), kc = (ci % (BK / VEC)) * VEC;
        const int m = m0 + row, k = k0 + kc;
        xr[t] = (m < M) ? load_vec_as<T>(P.A, P.a_dtype, (size_t)m * P.lda + k, K - k, P.vec_a)
                        : zero_vec<vec>();
      } else {
        const int kr = ci / (BM / VEC), mc = (ci % (BM / VEC)) * VEC;
        const int k = k0 + kr, m = m0 + mc;
        xr[t] = (k < K) ? load_vec_as<T>(P.A, P.a_dtype, (size_t)k * P.lda + m, M - m, P.vec_a)
                        : zero_vec<vec>();
      }
      if (!P.w_trans) {
        const int kr = ci / (BN / VEC), nc = (ci % (BN / VEC)) * VEC;
        const int k = k0 + kr, n = n0 + nc;
        wr[t] = (k < K) ? load_vec_as<T>(P.W, P.w_dtype, (size_t)k * P.ldw + n, N - n, P.vec_w)
                        : zero_vec<vec>();
      } else {
        const int row = ci / (BK / VEC), kc = (ci % (BK / VEC)) * VEC;
        const int n = n0 + row, k = k0 + kc;
        wr[t] = (n < N) ? load_vec_as<T>(P.W, P.w_dtype, (size_t)n * P.ldw + k, K - k, P.vec_w)
                        : zero_vec<vec>();
      }
    }
  };
  auto store_stage = [&]() {
    #pragma unroll
    for (int t = 0; t < PER_T; ++t) {
      const int ci = tid + t * NT;
      if (!P.a_trans) {
        const int row = ci / (BK / VEC), kc = (ci % (BK / VEC)) * VEC;
        *reinterpret_cast<vec*>(&Xs[row * PAD + kc]) = xr[t];
      } else {
        const int kr = ci / (BM / VEC), mc = (ci % (BM / VEC)) * VEC;
        #pragma unroll
        for (int e = 0; e < VEC; ++e) Xs[(mc + e) * PAD + kr] = xr[t][e];
      }
      if (!P.w_trans) {
        const int kr = ci / (BN / VEC), nc = (ci % (BN / VEC)) * VEC;
        #pragma unroll
        for (int e = 0; e < VEC; ++e) Wt[(nc + e) * PAD + kr] = wr[t][e];
      } else {
        const int row = ci / (BK / VEC), kc = (ci % (BK / VEC)) * VEC;
        *reinterpret_cast<vec*>(&Wt[row * PAD + kc]) = wr[t];
      }
    }
  };

  const int nstage = (K - kb + BK - 1) / BK;
  if (nstage > 0) load_stage(kb);
  for (int s = 0; s < nstage; ++s) {
    __syncthreads();
    store_stage();
    __syncthreads();
    if (s + 1 < nstage) load_stage(kb + (s + 1) * BK);
    #pragma unroll
    for (int kc = 0; kc < KCH; ++kc) {
      vec wf[2], xf[2];
      #pragma unroll
      for (int j = 0; j < 2; ++j)
        wf[j] = *reinterpret_cast<const vec*>(&Wt[(wn * WN + j * 32 + l32) * PAD + kc * 2 * VEC + g * VEC]);
      #pragma unroll
      for (int i = 0; i < 2; ++i)
        xf[i] = *reinterpret_cast<const vec*>(&Xs[(wm * WM + i * 32 + l32) * PAD + kc * 2 * VEC + g * VEC]);
      #pragma unroll
      for (int j = 0; j < 2; ++j)
        #pragma unroll
        for (int i = 0; i < 2; ++i) mfma_chunk(acc[j][i], wf[j], xf[i]);
    }
  }

  // acc[j][i]: rows m0 + wm*64 + 32 i + (lane % 32), columns
  // n0 + wn*64 + 32 j + 8 a + 4 g + (0..3) in registers 4a..4a+3
  #pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + wm * WM + i * 32 + l32;
    if (m >= M) continue;
    #pragma unroll
    for (int j = 0; j < 2; ++j)
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int n = n0 + wn * WN + j * 32 + 8 * a + 4 * g;
        if (n >= N) continue;
        if (P.ksplit > 1)
          store4(P.partial, kF32, ((size_t)ks * M + m) * N + n, (N % 4) == 0, N - n,
                 acc[j][i][4 * a], acc[j][i][4 * a + 1], acc[j][i][4 * a + 2], acc[j][i][4 * a + 3]);
        else
          store4(P.C, P.c_dtype, (size_t)m * P.ldc + n, P.vec_c, N - n, acc[j][i][4 * a],
                 acc[j][i][4 * a + 1], acc[j][i][4 * a + 2], acc[j][i][4 * a + 3]);
      }
  }
}

// Split-K: C[m, n] = sum over partitions s (in order) of partial[s, m, n].
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* partial, int S, int M,
                                                            int N, void* C, int c_dtype,
                                                            long long ldc) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t MN = (size_t)M * N;
  if (idx >= MN) return;
  float sum = 0.f;
  for (int s = 0; s < S; ++s) sum += partial[(size_t)s * MN + idx];
  const size_t m = idx / N, n = idx - m * N;
  const size_t o = m * ldc + n;
  if (c_dtype == kF32) reinterpret_cast<float*>(C)[o] = sum;
  else if (c_dtype == kBF16) reinterpret_cast<bf16*>(C)[o] = (bf16)sum;
  else reinterpret_cast<f16*>(C)[o] = (f16)sum;
}

// y[i] = x[i] rounded to y's element type (nearest even), fp32 source; each
// thread takes eight consecutive elements (two 16-byte loads, one 16-byte
// store when x and y are 16-byte aligned and all eight exist).
template <typename TY>
__global__ __launch_bounds__(256) void round_f32_kernel(const float* x, TY* y, size_t n,
                                                        int vec_ok) {
  typedef typename Elem<TY>::vec V;
  const size_t i0 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i0 >= n) return;
  if (vec_ok && i0 + 8 <= n) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(x + i0);
    const floatx4 b = *reinterpret_cast<const floatx4*>(x + i0 + 4);
    const floatx8 f = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    *reinterpret_cast<V*>(y + i0) = __builtin_convertvector(f, V);
  } else {
    for (size_t i = i0; i < n && i < i0 + 8; ++i) y[i] = (TY)x[i];
  }
}

// Column sums of a row-major [M, N] array of type dt (row stride ld): pass 1
// sums rows [256 r, 256 r + 256) of column n into part[r * N + n]; pass 2 sums
// the R partial rows into out[n] (type out_dtype).  Fixed order: deterministic.
__global__ __launch_bounds__(256) void colsum_partial_kernel(const void* X, int dt, long long ld,
                                                             int M, int N, float* part) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int r = blockIdx.y;
  if (n >= N) return;
  const int m1 = min(M, (r + 1) * 256);
  float s = 0.f;
  for (int m = r * 256; m < m1; ++m) {
    const size_t i = (size_t)m * ld + n;
    s += dt == kF32 ? reinterpret_cast<const float*>(X)[i]
         : dt == kBF16 ? (float)reinterpret_cast<const bf16*>(X)[i]
                       : (float)reinterpret_cast<const f16*>(X)[i];
  }
  part[(size_t)r * N + n] = s;
}

__global__ __launch_bounds__(256) void colsum_finish_kernel(const float* part, int R, int N,
                                                            void* out, int out_dtype) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  float s = 0.f;
  for (int r = 0; r < R; ++r) s += part[(size_t)r * N + n];
  if (out_dtype == kF32) reinterpret_cast<float*>(out)[n] = s;
  else if (out_dtype == kBF16) reinterpret_cast<bf16*>(out)[n] = (bf16)s;
  else reinterpret_cast<f16*>(out)[n] = (f16)s;
}

}  // namespace mha
