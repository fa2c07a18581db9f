// Device-side helpers shared by the libpoetx kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace poetx {

typedef uint16_t bf16_t;  // bfloat16 storage (bit pattern)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float floatx4;
typedef __attribute__((ext_vector_type(16))) float floatx16;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// float32 -> bfloat16, round to nearest even (NaN stays NaN): one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

template <typename T> struct ElemTraits;
template <> struct ElemTraits<float> {
  static constexpr int kVec = 4;  // elements per 16-byte vector
  __device__ static float to_f32(float v) { return v; }
  __device__ static float from_f32(float v) { return v; }
};
template <> struct ElemTraits<bf16_t> {
  static constexpr int kVec = 8;
  __device__ static float to_f32(bf16_t v) { return bf16_to_f32(v); }
  __device__ static bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

// Store a float32 value as T.
template <typename T>
__device__ __forceinline__ void store_as(T* p, float v) { *p = ElemTraits<T>::from_f32(v); }

}  // namespace poetx
