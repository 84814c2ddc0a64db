// Shared device helpers for the gfx950 kernels: element types, 16-byte
// vectors, the 32x32 MFMA step for each element type, conversions, stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mha {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;

// Element codes shared with the C ABI (mha_dtype).
enum DType : int { kF32 = 0, kBF16 = 1, kF16 = 2 };

// Element-type traits.  VEC = elements in one 16-byte vector; one "k-chunk"
// of a 32x32 MFMA step covers 2*VEC reduction indices (VEC per lane half).
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int VEC = 4;
  typedef floatx4 vec;
  typedef floatx4 vec4;
};
template <> struct Elem<bf16> {
  static constexpr int VEC = 8;
  typedef bf16x8 vec;
  typedef bf16x4 vec4;
};
template <> struct Elem<f16> {
  static constexpr int VEC = 8;
  typedef f16x8 vec;
  typedef f16x4 vec4;
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
__device__ __forceinline__ void mfma_chunk(floatx16& acc, const f16x8& a, const f16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_chunk(floatx16& acc, const floatx4& a, const floatx4& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b.w, acc, 0, 0, 0);
}

// Round-to-nearest-even conversions of fp32 vectors (hardware cvt_pk).
template <typename T> struct Cvt;
template <> struct Cvt<float> {
  __device__ __forceinline__ static floatx4 four(float a, float b, float c, float d) {
    floatx4 r = {a, b, c, d};
    return r;
  }
};
template <> struct Cvt<bf16> {
  __device__ __forceinline__ static bf16x4 four(float a, float b, float c, float d) {
    floatx4 v = {a, b, c, d};
    return __builtin_convertvector(v, bf16x4);
  }
  __device__ __forceinline__ static bf16x8 eight(const floatx8& v) {
    return __builtin_convertvector(v, bf16x8);
  }
};
template <> struct Cvt<f16> {
  __device__ __forceinline__ static f16x4 four(float a, float b, float c, float d) {
    floatx4 v = {a, b, c, d};
    return __builtin_convertvector(v, f16x4);
  }
  __device__ __forceinline__ static f16x8 eight(const floatx8& v) {
    return __builtin_convertvector(v, f16x8);
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

// A 16-byte chunk of one 2-byte type re-rounded to another (bf16 -> f16).
template <typename To, typename From>
__device__ __forceinline__ typename Elem<To>::vec convert_chunk(const typename Elem<From>::vec& v) {
  if constexpr (__is_same(To, From)) {
    return v;
  } else {
    floatx8 f = __builtin_convertvector(v, floatx8);
    return __builtin_convertvector(f, typename Elem<To>::vec);
  }
}

// Store up to four consecutive fp32 results at element offset `idx` of an
// array of element type `dtype` (DType), rounding to nearest even.  `count`
// is how many of the four are in range; `vec_ok` says a full store of four
// may be issued as one vector access (alignment checked by the caller).
__device__ __forceinline__ void store4(void* base, int dtype, size_t idx, bool vec_ok, int count,
                                       float v0, float v1, float v2, float v3) {
  if (count <= 0) return;
  if (dtype == kF32) {
    float* out = reinterpret_cast<float*>(base) + idx;
    if (vec_ok && count >= 4) {
      *reinterpret_cast<floatx4*>(out) = Cvt<float>::four(v0, v1, v2, v3);
    } else {
      const float v[4] = {v0, v1, v2, v3};
      for (int e = 0; e < 4 && e < count; ++e) out[e] = v[e];
    }
  } else if (dtype == kBF16) {
    bf16* out = reinterpret_cast<bf16*>(base) + idx;
    const bf16x4 pk = Cvt<bf16>::four(v0, v1, v2, v3);
    if (vec_ok && count >= 4) {
      *reinterpret_cast<bf16x4*>(out) = pk;
    } else {
      for (int e = 0; e < 4 && e < count; ++e) out[e] = pk[e];
    }
  } else {
    f16* out = reinterpret_cast<f16*>(base) + idx;
    const f16x4 pk = Cvt<f16>::four(v0, v1, v2, v3);
    if (vec_ok && count >= 4) {
      *reinterpret_cast<f16x4*>(out) = pk;
    } else {
      for (int e = 0; e < 4 && e < count; ++e) out[e] = pk[e];
    }
  }
}

// Transposing LDS read of four 16-bit values (gfx950 ds_read_b64_tr_b16).
// Within each group of 16 lanes, output lane i receives, in slot e, the
// value at position i % 4 of the four-element run addressed by lane
// 4e + i/4 of the same group (lane layout measured on the hardware).
template <typename T>
__device__ __forceinline__ typename Elem<T>::vec4 lds_read_tr4(const T* p) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s4*)(const_cast<T*>(p)));
  return __builtin_bit_cast(typename Elem<T>::vec4, v);
}

// LDS reads at a byte address (address space 3).  The kernels form one base
// per read pattern and block and add compile-time offsets, which the
// instructions take as immediates.
template <typename V>
__device__ __forceinline__ V lds_load_at(unsigned addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) V*>(addr);
}
template <typename T>
__device__ __forceinline__ typename Elem<T>::vec4 lds_read_tr4_at(unsigned addr) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  const s4 v =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<__attribute__((address_space(3))) s4*>(addr));
  return __builtin_bit_cast(typename Elem<T>::vec4, v);
}

// Combine a per-lane value with the lane 32 positions away (the other half
// of the wave).  v_permlane32_swap exchanges the halves of two registers;
// with both operands equal, the two results hold the lower half's and the
// upper half's values on every lane, in one order or the other.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace mha
