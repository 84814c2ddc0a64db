// Shared device helpers for the gfx950 kernels: element types, 16-byte
// vectors, the 32x32 MFMA step for each element type, conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mha {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element-type traits.  VEC = elements in one 16-byte vector; one "k-chunk"
// of a 32x32 MFMA step covers 2*VEC reduction indices (VEC per lane half).
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int VEC = 4;
  typedef floatx4 vec;
};
template <> struct Elem<bf16> {
  static constexpr int VEC = 8;
  typedef bf16x8 vec;
};

// acc += A(32 x kchunk) * B(kchunk x 32) on the matrix cores.
// Lane l supplies row (l % 32) of A and column (l % 32) of B; lane half
// g = l / 32 supplies VEC reduction indices.  The pairing of reduction
// indices between A and B is the same in both operands, so any fixed
// assignment of k values to (half, slot) gives the full sum.
// Result layout (32x32, fp32): acc[i] holds row 8*(i/4) + 4*g + (i%4),
// column l % 32.
__device__ __forceinline__ void mfma_chunk(floatx16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_chunk(floatx16& acc, const floatx4& a, const floatx4& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b.w, acc, 0, 0, 0);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Four fp32 values -> four elements of T, round to nearest even.
template <typename T> struct Pack4;
template <> struct Pack4<float> {
  typedef floatx4 type;
  __device__ __forceinline__ static floatx4 make(float a, float b, float c, float d) {
    floatx4 r = {a, b, c, d};
    return r;
  }
};
template <> struct Pack4<bf16> {
  typedef bf16x4 type;
  __device__ __forceinline__ static bf16x4 make(float a, float b, float c, float d) {
    floatx2 lo = {a, b}, hi = {c, d};
    bf16x2 l2 = __builtin_convertvector(lo, bf16x2);
    bf16x2 h2 = __builtin_convertvector(hi, bf16x2);
    bf16x4 r = {l2.x, l2.y, h2.x, h2.y};
    return r;
  }
};

template <typename V> __device__ __forceinline__ V zero_vec() {
  V v;
  #pragma unroll
  for (int i = 0; i < (int)(sizeof(V) / sizeof(v[0])); ++i) v[i] = 0;
  return v;
}

// Load VEC consecutive elements starting at column `col` of a row of `ncols`
// valid elements.  `vec_ok`: the row base is 16-byte aligned and the row
// stride is a multiple of VEC, so a full in-range chunk may be loaded as one
// 16-byte access.  Elements at or past `ncols` read as zero.
template <typename T>
__device__ __forceinline__ typename Elem<T>::vec load_chunk(const T* __restrict__ row, int col,
                                                            int ncols, bool vec_ok) {
  typedef typename Elem<T>::vec V;
  constexpr int VEC = Elem<T>::VEC;
  if (vec_ok && col + VEC <= ncols) {
    return *reinterpret_cast<const V*>(row + col);
  }
  V v = zero_vec<V>();
  #pragma unroll
  for (int e = 0; e < VEC; ++e)
    if (col + e < ncols) v[e] = row[col + e];
  return v;
}

// Store up to four consecutive fp32 results at element offset `idx` of an
// fp32 or bf16 array (`dtype` 0 = fp32, 1 = bf16), rounding to nearest even.
// `count` is how many of the four are in range; `vec_ok` says a full store
// of four may be issued as one vector access (alignment checked by caller).
__device__ __forceinline__ void store4(void* base, int dtype, size_t idx, bool vec_ok, int count,
                                       float v0, float v1, float v2, float v3) {
  if (count <= 0) return;
  if (dtype == 0) {
    float* out = reinterpret_cast<float*>(base) + idx;
    if (vec_ok && count >= 4) {
      *reinterpret_cast<floatx4*>(out) = Pack4<float>::make(v0, v1, v2, v3);
    } else {
      const float v[4] = {v0, v1, v2, v3};
      for (int e = 0; e < 4 && e < count; ++e) out[e] = v[e];
    }
  } else {
    bf16* out = reinterpret_cast<bf16*>(base) + idx;
    const bf16x4 pk = Pack4<bf16>::make(v0, v1, v2, v3);
    if (vec_ok && count >= 4) {
      *reinterpret_cast<bf16x4*>(out) = pk;
    } else {
      for (int e = 0; e < 4 && e < count; ++e) out[e] = pk[e];
    }
  }
}

__device__ __forceinline__ float wave_xor32(float x) {
  // exchange with the lane 32 positions away (the other half of the wave)
  return __shfl_xor(x, 32, 64);
}

}  // namespace mha
