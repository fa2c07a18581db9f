// INT8 frozen weight (POET-XQ): per-row quantisation, exact dequantisation of
// the codes, and the column-scaled R blocks that carry the row scales.
//
// Method (gist.science technical summary of "POET-X: Memory-efficient LLM
// Training by Scaling Orthogonal Transformation", section 2 Methodik,
// quantised-support item): because the orthogonal transform acts on the
// activations and no high-precision copy of the weight must be kept, the
// frozen weight can be an INT8 model. Scheme (not stated on the pages):
// symmetric, one float32 scale per output row, s_i = amax_i / 127,
// q_ij = clamp(rint(w_ij / s_i), -127, 127), both divisions correctly rounded
// in float32; W0 = diag(s) q.
//
// The layer never forms diag(s) q in bf16 (that would round it): the codes
// are widened to bf16 exactly (|q| <= 127), the products run on the codes,
// and s enters through the R side, Y = (U q^T) (R diag(s))^T and
// g_Z' = g_Y R diag(s), g_U = g_Z' q, G_R = (g_Y^T (U q^T)) diag(s).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace poetx {
namespace {

constexpr int kNT = 256;

template <typename T> struct In8;  // 8 activation-type values (16 or 32 bytes)
template <> struct In8<bf16_t> {
  static __device__ void load(const bf16_t* p, float v[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v[2 * t] = __uint_as_float(w[t] << 16);
      v[2 * t + 1] = __uint_as_float(w[t] & 0xffff0000u);
    }
  }
};
template <> struct In8<float> {
  static __device__ void load(const float* p, float v[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

// One workgroup per row (striding): amax by a wave then workgroup max, then
// the codes. d_in % 8 == 0.
template <typename T>
__global__ void __launch_bounds__(kNT)
quantize_rows_kernel(const T* __restrict__ W, int64_t rows, int d, int8_t* __restrict__ q,
                     float* __restrict__ scale) {
  __shared__ float wmax[kNT / 64];
  const int nv = d / 8;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const T* row = W + r * d;
    float m = 0.0f;
    for (int c = threadIdx.x; c < nv; c += kNT) {
      float v[8];
      In8<T>::load(row + 8 * c, v);
#pragma unroll
      for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(v[t]));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    __syncthreads();  // wmax of the previous row has been read
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    float amax = wmax[0];
#pragma unroll
    for (int w = 1; w < kNT / 64; ++w) amax = fmaxf(amax, wmax[w]);
    const float s = __fdiv_rn(amax, 127.0f);
    if (threadIdx.x == 0) scale[r] = s;
    int8_t* qr = q + r * d;
    for (int c = threadIdx.x; c < nv; c += kNT) {
      float v[8];
      In8<T>::load(row + 8 * c, v);
      union { uint2 u; int8_t b[8]; } o;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        float x = 0.0f;
        if (s > 0.0f) x = fminf(fmaxf(rintf(__fdiv_rn(v[t], s)), -127.0f), 127.0f);
        o.b[t] = (int8_t)(int)x;
      }
      *reinterpret_cast<uint2*>(qr + 8 * c) = o.u;
    }
  }
}

// out = (activation type) q, exact; n % 8 == 0.
template <typename T>
__global__ void __launch_bounds__(kNT)
widen_codes_kernel(const int8_t* __restrict__ q, int64_t ldq, int64_t cols8, int64_t n8,
                   T* __restrict__ out) {
  // group i: row i / cols8, codes 8 (i % cols8) .. + 7 of the slice (the
  // slice's rows are ldq codes apart in q, cols8 groups apart in out)
  for (int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x; i < n8; i += (int64_t)gridDim.x * kNT) {
    const int64_t r = i / cols8, g = i - r * cols8;
    union { uint2 u; int8_t b[8]; } in;
    in.u = *reinterpret_cast<const uint2*>(q + r * ldq + 8 * g);
    if constexpr (sizeof(T) == 2) {
      union { uint4 u; bf16_t h[8]; } o;
#pragma unroll
      for (int t = 0; t < 8; ++t) o.h[t] = f32_to_bf16((float)in.b[t]);
      reinterpret_cast<uint4*>(out)[i] = o.u;
    } else {
      float4 a, b;
      a.x = in.b[0]; a.y = in.b[1]; a.z = in.b[2]; a.w = in.b[3];
      b.x = in.b[4]; b.y = in.b[5]; b.z = in.b[6]; b.w = in.b[7];
      reinterpret_cast<float4*>(out)[2 * i] = a;
      reinterpret_cast<float4*>(out)[2 * i + 1] = b;
    }
  }
}

// The same into the tiled layout (bf16; rows % 256 == 0, cols % 32 == 0),
// walked in the output's order so that the stores are contiguous: group i
// is the 8 codes at (r, k) of 256 x 32 block i / 1024, whose rows are 4
// groups each.
__global__ void __launch_bounds__(kNT)
widen_codes_tiled_kernel(const int8_t* __restrict__ q, int64_t ldq, int64_t kblocks, int64_t n8,
                         bf16_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * kNT + threadIdx.x; i < n8; i += (int64_t)gridDim.x * kNT) {
    const int64_t blk = i >> 10, rb = blk / kblocks;
    const int64_t r = rb * 256 + ((i >> 2) & 255);
    const int64_t k = (blk - rb * kblocks) * 32 + (i & 3) * 8;
    union { uint2 u; int8_t b[8]; } in;
    in.u = *reinterpret_cast<const uint2*>(q + r * ldq + k);
    union { uint4 u; bf16_t h[8]; } o;
#pragma unroll
    for (int t = 0; t < 8; ++t) o.h[t] = f32_to_bf16((float)in.b[t]);
    reinterpret_cast<uint4*>(out)[i] = o.u;
  }
}

// out[k][i][j] = M[k][i][j] * s[k b + j] (0 for columns past d), in the
// activation type. Flat over nblocks * b * b.
template <typename T>
__global__ void __launch_bounds__(kNT)
scale_block_columns_kernel(const T* __restrict__ M, const float* __restrict__ s, int64_t total,
                           int b, int64_t d, T* __restrict__ out) {
  const int64_t bb = (int64_t)b * b;
  for (int64_t e = (int64_t)blockIdx.x * kNT + threadIdx.x; e < total; e += (int64_t)gridDim.x * kNT) {
    const int64_t k = e / bb;
    const int j = (int)(e % b);
    const int64_t col = k * b + j;
    const float sc = col < d ? s[col] : 0.0f;
    if constexpr (sizeof(T) == 2)
      out[e] = f32_to_bf16(bf16_to_f32(M[e]) * sc);
    else
      out[e] = M[e] * sc;
  }
}

// The same for b % 4 == 0, grid (ceil(b b / (4 kNT)), nblocks): each thread
// scales four consecutive columns of one row (they never straddle a row), with
// 32-bit index arithmetic inside the block.
__device__ __forceinline__ void scale4(const float* in, float* out, const float sc[4]) {
  const float4 v = *reinterpret_cast<const float4*>(in);
  *reinterpret_cast<float4*>(out) = make_float4(v.x * sc[0], v.y * sc[1], v.z * sc[2], v.w * sc[3]);
}
__device__ __forceinline__ void scale4(const bf16_t* in, bf16_t* out, const float sc[4]) {
  union { uint2 u; bf16_t h[4]; } v;
  v.u = *reinterpret_cast<const uint2*>(in);
#pragma unroll
  for (int t = 0; t < 4; ++t) v.h[t] = f32_to_bf16(bf16_to_f32(v.h[t]) * sc[t]);
  *reinterpret_cast<uint2*>(out) = v.u;
}
template <typename T>
__global__ void __launch_bounds__(kNT)
scale_block_columns4_kernel(const T* __restrict__ M, const float* __restrict__ s, int b, int64_t d,
                            T* __restrict__ out) {
  const int q = (int)blockIdx.x * kNT + (int)threadIdx.x;
  if (q >= b * b / 4) return;
  const int e = 4 * q, j = e % b;
  const int64_t base = (int64_t)blockIdx.y * b * b + e;
  const int64_t col = (int64_t)blockIdx.y * b + j;
  float sc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) sc[t] = col + t < d ? s[col + t] : 0.0f;
  scale4(M + base, out + base, sc);
}

int flat_grid(int64_t n) { return (int)std::min<int64_t>((n + kNT - 1) / kNT, 8192); }

}  // namespace

hipError_t launch_quantize_rows(DType t, const void* W, int64_t rows, int d, int8_t* q,
                                float* scale, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>(rows, 4096);
  if (t == DType::BF16)
    hipLaunchKernelGGL(quantize_rows_kernel<bf16_t>, dim3(grid), dim3(kNT), 0, s,
                       static_cast<const bf16_t*>(W), rows, d, q, scale);
  else
    hipLaunchKernelGGL(quantize_rows_kernel<float>, dim3(grid), dim3(kNT), 0, s,
                       static_cast<const float*>(W), rows, d, q, scale);
  return hipGetLastError();
}

hipError_t launch_widen_codes(DType t, const int8_t* q, int64_t rows, int64_t ldq, int64_t cols,
                              void* out, bool out_tiled, hipStream_t s) {
  if (cols % 8 != 0 || ldq % 8 != 0 || cols > ldq || rows < 0) return hipErrorInvalidValue;
  if (out_tiled && (t != DType::BF16 || rows % 256 != 0 || cols % 32 != 0))
    return hipErrorInvalidValue;
  const int64_t n8 = rows * (cols / 8);
  if (n8 == 0) return hipSuccess;
  if (out_tiled)
    hipLaunchKernelGGL(widen_codes_tiled_kernel, dim3(flat_grid(n8)), dim3(kNT), 0, s, q, ldq,
                       cols / 32, n8, static_cast<bf16_t*>(out));
  else if (t == DType::BF16)
    hipLaunchKernelGGL(widen_codes_kernel<bf16_t>, dim3(flat_grid(n8)), dim3(kNT), 0, s, q, ldq,
                       cols / 8, n8, static_cast<bf16_t*>(out));
  else
    hipLaunchKernelGGL(widen_codes_kernel<float>, dim3(flat_grid(n8)), dim3(kNT), 0, s, q, ldq,
                       cols / 8, n8, static_cast<float*>(out));
  return hipGetLastError();
}

hipError_t launch_scale_block_columns(DType t, const void* M, const float* scale, int64_t nblocks,
                                      int b, int64_t d, void* out, hipStream_t s) {
  const int64_t total = nblocks * b * b;
  if (total == 0) return hipSuccess;
  if (b % 4 == 0 && nblocks <= 65535) {
    const dim3 grid((unsigned)((b * b / 4 + kNT - 1) / kNT), (unsigned)nblocks);
    if (t == DType::BF16)
      hipLaunchKernelGGL(scale_block_columns4_kernel<bf16_t>, grid, dim3(kNT), 0, s,
                         static_cast<const bf16_t*>(M), scale, b, d, static_cast<bf16_t*>(out));
    else
      hipLaunchKernelGGL(scale_block_columns4_kernel<float>, grid, dim3(kNT), 0, s,
                         static_cast<const float*>(M), scale, b, d, static_cast<float*>(out));
    return hipGetLastError();
  }
  if (t == DType::BF16)
    hipLaunchKernelGGL(scale_block_columns_kernel<bf16_t>, dim3(flat_grid(total)), dim3(kNT), 0, s,
                       static_cast<const bf16_t*>(M), scale, total, b, d, static_cast<bf16_t*>(out));
  else
    hipLaunchKernelGGL(scale_block_columns_kernel<float>, dim3(flat_grid(total)), dim3(kNT), 0, s,
                       static_cast<const float*>(M), scale, total, b, d, static_cast<float*>(out));
  return hipGetLastError();
}

}  // namespace poetx
