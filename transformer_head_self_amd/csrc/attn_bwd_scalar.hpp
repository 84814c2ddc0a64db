// Vector-ALU kernels of the attention backward (any element type of the
// heads; fp32 accumulation), and the gradient with respect to an additive
// score bias.
//
// Same mathematics as attn_bwd.hpp (calculus on the forward of page
// "Multi-head attention and self-attention", Definition; the weights
// recomputed from the forward's row statistics as page "Stable summary of an
// attention key block", Definition, gives them):
//   dV = A^T dZ,  dA = dZ V^T,  dS = A o (dA - D),  dQ = c dS K,  dK = c dS^T Q,
// and, for scores S = c Q K^T + M with one bias M for every head,
//   dM = sum over heads of dS (and over the batch items when one M serves
//   them all).
// The matrix-core kernels take 2-byte heads; these take fp32 heads too
// (fp32 operands, no rounding) and form dM, which the matrix-core kernels
// cannot: it sums over heads, while their grids give each head its own
// workgroups.  Layout of the work (ours): four lanes (a quad) share one
// row of the 64-row tile a workgroup owns and split its d columns four
// ways; a dot product is the quad's partial sums added with two DPP quad
// permutes.  The other operand's rows stream through LDS as fp32, 64 rows
// at a time, and every lane of the workgroup walks them in the same order,
// so the sums have a fixed order (deterministic).
#pragma once

#include "attn_bwd.hpp"

namespace mha {

// Sum over the four lanes of a quad (DPP quad permutes [1,0,3,2], [2,3,0,1]).
__device__ __forceinline__ float quad_sum(float x) {
  int xi = __builtin_bit_cast(int, x);
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, xi, 0xB1, 0xF, 0xF, false));
  xi = __builtin_bit_cast(int, x);
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, xi, 0x4E, 0xF, 0xF, false));
  return x;
}

__device__ __forceinline__ void store1(void* base, int dtype, size_t idx, float v) {
  if (dtype == kF32) reinterpret_cast<float*>(base)[idx] = v;
  else if (dtype == kBF16) reinterpret_cast<bf16*>(base)[idx] = (bf16)v;
  else reinterpret_cast<f16*>(base)[idx] = (f16)v;
}

// Stage rows r0 .. r0 + 63 (of nrows) and columns 0 .. ncols - 1 (of D) of a
// row-major array into an fp32 LDS tile, each value rounded to round_to (2-byte
// heads take dZ rounded to their type, as the row term D does); rows and
// columns past the end are 0.
template <int D>
__device__ __forceinline__ void stage_rows_f32(float (*tile)[D + 1], const void* base, int dtype,
                                               size_t off, size_t ld, int r0, int nrows, int ncols,
                                               int round_to, int tid) {
  for (int idx = tid; idx < 64 * D; idx += 256) {
    const int rr = idx / D, cc = idx - rr * D;
    float v = 0.f;
    if (r0 + rr < nrows && cc < ncols)
      v = round_as(load1_as(base, dtype, off + (size_t)(r0 + rr) * ld + cc), round_to);
    tile[rr][cc] = v;
  }
}

// dK, dV: one workgroup per (64 keys, b*h + r); quad jl = tid / 4 owns key
// k0 + jl, lane part = tid % 4 its columns part*DH/4 .. (and DV/4).
template <int DH, int DV>
__global__ __launch_bounds__(256) void attn_bwd_kv_scalar_kernel(AttnBwdParams p) {
  constexpr int SH = DH / 4, SV = DV / 4;
  __shared__ float Qs[64][DH + 1];
  __shared__ float Zs[64][DV + 1];
  __shared__ float Ls[64], Ds[64];
  const int tid = threadIdx.x, jl = tid >> 2, part = tid & 3;
  const int BH = p.B * p.h;
  const int kt = blockIdx.x / BH, bh = blockIdx.x - kt * BH;
  const int b = bh / p.h, r = bh - b * p.h;
  const int k0 = kt * 64, key = k0 + jl;
  int kvalid = p.n_k;
  if (p.key_len) kvalid = min(kvalid, p.key_len[b]);
  const uint8_t* G = p.allowed ? p.allowed + (size_t)b * p.allowed_batch_stride : nullptr;
  const float* M = p.add ? p.add + (size_t)b * p.add_batch_stride : nullptr;

  float kr[SH], vr[SV], dk[SH], dv[SV];
  #pragma unroll
  for (int e = 0; e < SH; ++e) {
    const int c = part * SH + e;
    kr[e] = (key < p.n_k && c < p.d_h)
                ? load1_as(p.K, p.elem_dtype, ((size_t)bh * p.n_k + key) * p.d_h + c) : 0.f;
    dk[e] = 0.f;
  }
  #pragma unroll
  for (int e = 0; e < SV; ++e) {
    const int c = part * SV + e;
    vr[e] = (key < p.n_k && c < p.d_vh)
                ? load1_as(p.V, p.elem_dtype, ((size_t)bh * p.n_k + key) * p.d_vh + c) : 0.f;
    dv[e] = 0.f;
  }
  // a causal key k sees queries q >= k: start at the tile's first key; a
  // tile wholly past the item's keys sees none
  const int qbeg = p.causal ? k0 : 0;
  const int qend = k0 < kvalid ? p.n_q : qbeg;
  for (int q0 = qbeg; q0 < qend; q0 += 64) {
    __syncthreads();
    stage_rows_f32<DH>(Qs, p.Q, p.elem_dtype, (size_t)bh * p.n_q * p.d_h, p.d_h, q0, p.n_q,
                       p.d_h, kF32, tid);
    stage_rows_f32<DV>(Zs, p.dZ, p.z_dtype, (size_t)b * p.n_q * p.ldz + (size_t)r * p.d_vh,
                       p.ldz, q0, p.n_q, p.d_vh, p.elem_dtype, tid);
    if (tid < 64) {
      const int q = q0 + tid;
      Ls[tid] = q < p.n_q ? p.lse2[(size_t)bh * p.n_q + q] : INFINITY;
      Ds[tid] = q < p.n_q ? p.dsum[(size_t)bh * p.n_q + q] : 0.f;
    }
    __syncthreads();
    const int nq = min(64, p.n_q - q0);
    for (int i = 0; i < nq; ++i) {
      const int q = q0 + i;
      float s = 0.f, da = 0.f;
      #pragma unroll
      for (int e = 0; e < SH; ++e) s = fmaf(Qs[i][part * SH + e], kr[e], s);
      #pragma unroll
      for (int e = 0; e < SV; ++e) da = fmaf(Zs[i][part * SV + e], vr[e], da);
      s = quad_sum(s);
      da = quad_sum(da);
      const bool ok = bwd_allowed(p, G, q, key, kvalid);
      float x = s * p.scale_log2;
      if (M != nullptr && ok) x = fmaf(M[(size_t)q * p.n_k + key], kLog2e, x);
      const float a = ok ? __builtin_amdgcn_exp2f(x - Ls[i]) : 0.f;
      const float ds = a * (da - Ds[i]);
      #pragma unroll
      for (int e = 0; e < SV; ++e) dv[e] = fmaf(a, Zs[i][part * SV + e], dv[e]);
      #pragma unroll
      for (int e = 0; e < SH; ++e) dk[e] = fmaf(ds, Qs[i][part * SH + e], dk[e]);
    }
  }
  if (key < p.n_k) {
    const size_t kro = (p.grad_concat ? ((size_t)b * p.n_k + key) * p.h + r
                                      : (size_t)bh * p.n_k + key);
    #pragma unroll
    for (int e = 0; e < SH; ++e) {
      const int c = part * SH + e;
      if (c < p.d_h) store1(p.dK, p.g_dtype, kro * p.d_h + c, dk[e] * p.scale);
    }
    #pragma unroll
    for (int e = 0; e < SV; ++e) {
      const int c = part * SV + e;
      if (c < p.d_vh) store1(p.dV, p.g_dtype, kro * p.d_vh + c, dv[e]);
    }
  }
}

// dQ: one workgroup per (64 queries, b*h + r); quad il = tid / 4 owns query
// q0 + il.
template <int DH, int DV>
__global__ __launch_bounds__(256) void attn_bwd_q_scalar_kernel(AttnBwdParams p) {
  constexpr int SH = DH / 4, SV = DV / 4;
  __shared__ float Ks[64][DH + 1];
  __shared__ float Vs[64][DV + 1];
  const int tid = threadIdx.x, il = tid >> 2, part = tid & 3;
  const int BH = p.B * p.h;
  const int qt = blockIdx.x / BH, bh = blockIdx.x - qt * BH;
  const int b = bh / p.h, r = bh - b * p.h;
  const int q0 = qt * 64, q = q0 + il;
  int kvalid = p.n_k;
  if (p.key_len) kvalid = min(kvalid, p.key_len[b]);
  int kend = kvalid;
  if (p.causal) kend = min(kend, q0 + 64);
  const uint8_t* G = p.allowed ? p.allowed + (size_t)b * p.allowed_batch_stride : nullptr;
  const float* M = p.add ? p.add + (size_t)b * p.add_batch_stride : nullptr;

  float qr[SH], zr[SV], dq[SH];
  const size_t zrow = ((size_t)b * p.n_q + q) * p.ldz + (size_t)r * p.d_vh;
  #pragma unroll
  for (int e = 0; e < SH; ++e) {
    const int c = part * SH + e;
    qr[e] = (q < p.n_q && c < p.d_h)
                ? load1_as(p.Q, p.elem_dtype, ((size_t)bh * p.n_q + q) * p.d_h + c) : 0.f;
    dq[e] = 0.f;
  }
  #pragma unroll
  for (int e = 0; e < SV; ++e) {
    const int c = part * SV + e;
    zr[e] = (q < p.n_q && c < p.d_vh)
                ? round_as(load1_as(p.dZ, p.z_dtype, zrow + c), p.elem_dtype) : 0.f;
  }
  const float L = q < p.n_q ? p.lse2[(size_t)bh * p.n_q + q] : INFINITY;
  const float D = q < p.n_q ? p.dsum[(size_t)bh * p.n_q + q] : 0.f;

  for (int k0 = 0; k0 < kend; k0 += 64) {
    __syncthreads();
    stage_rows_f32<DH>(Ks, p.K, p.elem_dtype, (size_t)bh * p.n_k * p.d_h, p.d_h, k0, p.n_k,
                       p.d_h, kF32, tid);
    stage_rows_f32<DV>(Vs, p.V, p.elem_dtype, (size_t)bh * p.n_k * p.d_vh, p.d_vh, k0, p.n_k,
                       p.d_vh, kF32, tid);
    __syncthreads();
    const int nk = min(64, kend - k0);
    for (int j = 0; j < nk; ++j) {
      const int key = k0 + j;
      float s = 0.f, da = 0.f;
      #pragma unroll
      for (int e = 0; e < SH; ++e) s = fmaf(qr[e], Ks[j][part * SH + e], s);
      #pragma unroll
      for (int e = 0; e < SV; ++e) da = fmaf(zr[e], Vs[j][part * SV + e], da);
      s = quad_sum(s);
      da = quad_sum(da);
      const bool ok = bwd_allowed(p, G, q, key, kvalid);
      float x = s * p.scale_log2;
      if (M != nullptr && ok) x = fmaf(M[(size_t)q * p.n_k + key], kLog2e, x);
      const float a = ok ? __builtin_amdgcn_exp2f(x - L) : 0.f;
      const float ds = a * (da - D);
      #pragma unroll
      for (int e = 0; e < SH; ++e) dq[e] = fmaf(ds, Ks[j][part * SH + e], dq[e]);
    }
  }
  if (q < p.n_q) {
    const size_t qro = (p.grad_concat ? ((size_t)b * p.n_q + q) * p.h + r
                                      : (size_t)bh * p.n_q + q);
    #pragma unroll
    for (int e = 0; e < SH; ++e) {
      const int c = part * SH + e;
      if (c < p.d_h) store1(p.dQ, p.g_dtype, qro * p.d_h + c, dq[e] * p.scale);
    }
  }
}

// dM [Bo, n_q, n_k] (fp32; Bo = B, or 1 when one bias serves every item):
// one workgroup per (64 queries, output item, 64 keys); quad il owns query
// q0 + il, and after the quad's sums every lane of it holds dS for each
// key, of which lane part keeps keys k0 + 4 jj + part.  Heads (and items,
// for a shared bias) are visited in order, so the sum over them is formed
// in a fixed order.  Blocks no query may use are written as 0.
template <int DH, int DV>
__global__ __launch_bounds__(256) void attn_bwd_dm_kernel(AttnBwdParams p, float* dM,
                                                          int shared_bias) {
  constexpr int SH = DH / 4, SV = DV / 4;
  __shared__ float Ks[64][DH + 1];
  __shared__ float Vs[64][DV + 1];
  const int tid = threadIdx.x, il = tid >> 2, part = tid & 3;
  const int nkt = (p.n_k + 63) / 64;
  const int Bo = shared_bias ? 1 : p.B;
  const int kt = blockIdx.x % nkt;
  const int rest = blockIdx.x / nkt;
  const int bo = rest % Bo, qt = rest / Bo;
  const int q0 = qt * 64, q = q0 + il, k0 = kt * 64;
  const int nk = min(64, p.n_k - k0);

  float dm[16];
  #pragma unroll
  for (int jj = 0; jj < 16; ++jj) dm[jj] = 0.f;

  const int b_lo = shared_bias ? 0 : bo, b_hi = shared_bias ? p.B : bo + 1;
  const bool tile_live = !(p.causal && k0 > q0 + 63);
  for (int b = b_lo; b < b_hi && tile_live; ++b) {
    int kvalid = p.n_k;
    if (p.key_len) kvalid = min(kvalid, p.key_len[b]);
    if (k0 >= kvalid) continue;
    const uint8_t* G = p.allowed ? p.allowed + (size_t)b * p.allowed_batch_stride : nullptr;
    const float* M = p.add + (size_t)b * p.add_batch_stride;
    for (int r = 0; r < p.h; ++r) {
      const int bh = b * p.h + r;
      float qr[SH], zr[SV];
      const size_t zrow = ((size_t)b * p.n_q + q) * p.ldz + (size_t)r * p.d_vh;
      #pragma unroll
      for (int e = 0; e < SH; ++e) {
        const int c = part * SH + e;
        qr[e] = (q < p.n_q && c < p.d_h)
                    ? load1_as(p.Q, p.elem_dtype, ((size_t)bh * p.n_q + q) * p.d_h + c) : 0.f;
      }
      #pragma unroll
      for (int e = 0; e < SV; ++e) {
        const int c = part * SV + e;
        zr[e] = (q < p.n_q && c < p.d_vh)
                    ? round_as(load1_as(p.dZ, p.z_dtype, zrow + c), p.elem_dtype) : 0.f;
      }
      const float L = q < p.n_q ? p.lse2[(size_t)bh * p.n_q + q] : INFINITY;
      const float D = q < p.n_q ? p.dsum[(size_t)bh * p.n_q + q] : 0.f;
      __syncthreads();
      stage_rows_f32<DH>(Ks, p.K, p.elem_dtype, (size_t)bh * p.n_k * p.d_h, p.d_h, k0, p.n_k,
                         p.d_h, kF32, tid);
      stage_rows_f32<DV>(Vs, p.V, p.elem_dtype, (size_t)bh * p.n_k * p.d_vh, p.d_vh, k0, p.n_k,
                         p.d_vh, kF32, tid);
      __syncthreads();
      #pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        #pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = 4 * jj + u;
          if (j < nk) {
            const int key = k0 + j;
            float s = 0.f, da = 0.f;
            #pragma unroll
            for (int e = 0; e < SH; ++e) s = fmaf(qr[e], Ks[j][part * SH + e], s);
            #pragma unroll
            for (int e = 0; e < SV; ++e) da = fmaf(zr[e], Vs[j][part * SV + e], da);
            s = quad_sum(s);
            da = quad_sum(da);
            const bool ok = bwd_allowed(p, G, q, key, kvalid);
            float x = s * p.scale_log2;
            if (ok) x = fmaf(M[(size_t)q * p.n_k + key], kLog2e, x);
            const float a = ok ? __builtin_amdgcn_exp2f(x - L) : 0.f;
            const float ds = a * (da - D);
            dm[jj] += (u == part) ? ds : 0.f;
          }
        }
      }
    }
  }
  if (q < p.n_q) {
    float* row = dM + ((size_t)bo * p.n_q + q) * p.n_k;
    #pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const int key = k0 + 4 * jj + part;
      if (4 * jj + part < nk) row[key] = dm[jj];
    }
  }
}

}  // namespace mha
