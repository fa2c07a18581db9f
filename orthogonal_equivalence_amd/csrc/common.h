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

// Output tile (mt, nt) of this workgroup in a num_mt x num_nt grid.
// Workgroups are dispatched round-robin over the 8 XCDs; the order is
// remapped so each XCD works on a contiguous range of a grouped ordering
// (GROUP_M row tiles at a time), which keeps the operand panels that
// concurrently running tiles share in that XCD's L2.
// The index form maps logical workgroup wg of nwg (a persistent workgroup
// that walks wg, wg + G, ... with G a multiple of 8 stays on one XCD).
__device__ __forceinline__ void xcd_grouped_tile_at(int wg, int nwg, int num_mt, int num_nt, int& mt,
                                                    int& nt) {
  constexpr int GROUP_M = 8;
  if ((nwg & 7) == 0) wg = (wg & 7) * (nwg >> 3) + (wg >> 3);
  const int per_group = GROUP_M * num_nt;
  const int group = wg / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(num_mt - first_m, GROUP_M);
  const int in_group = wg - group * per_group;
  mt = first_m + in_group % gsize;
  nt = in_group / gsize;
}
__device__ __forceinline__ void xcd_grouped_tile(int num_mt, int num_nt, int& mt, int& nt) {
  xcd_grouped_tile_at(blockIdx.x, gridDim.x, num_mt, num_nt, mt, nt);
}

// Store a float32 value as T.
template <typename T>
__device__ __forceinline__ void store_as(T* p, float v) { *p = ElemTraits<T>::from_f32(v); }

}  // namespace poetx
