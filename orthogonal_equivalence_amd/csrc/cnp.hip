// Cayley-Neumann series variant of the orthogonal map: the elementwise
// steps of the build and of its VJP. The b x b products run on the batched
// MFMA GEMM: float32 for the build, and for the VJP float32 or (bf16
// activations) bf16 operands with float32 accumulation.
//
// Method (gist.science technical summary of "POET-X: Memory-efficient LLM
// Training by Scaling Orthogonal Transformation", section 2 Methodik,
// Cayley-Neumann parameterisation item): the Cayley map of a skew Q is
// approximated by a truncated Neumann series with the higher-order terms
// Q^2, Q^3, Q^4. Truncating (I - Q)^-1 inside R = 2 (I - Q)^-1 - I gives
//   R = I + 2 (Q + Q^2 + Q^3 + Q^4),
// built with two dependent products instead of three:
//   Q2 = Q Q,   E = Q2 Q2 + Q2,   F = Q Q2 + Q   (E and F in one launch),
//   R  = I + 2 (E + F)                           (cnp_finish_kernel).
// The pages fuse Q^2..Q^4 into one kernel with Q and Q^2 held in shared
// memory; at b = 256 in float32 each of them is 256 KB, more than a CU's
// LDS, so here the products are batched GEMM launches over all blocks.
//
// VJP, for G = dL/dR (chain rule of the series, in factored form): with
// T = Q + Q2 and N = I + Q2, R = I + 2 T N, so
//   Tbar = 2 G N = 2 G Q2 + 2 G,   Nbar = 2 T^T G = 2 (Q2 - Q) G,
//   dL/dQ = Tbar - W Q - Q W,      W = Tbar + Nbar,
// and since Q is skew, the packed gradient dL/dQ[i][j] - dL/dQ[j][i] equals
// X[i][j] - X[j][i] for X = Tbar - (W + W^T) Q.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace poetx {
namespace {

constexpr int kNT = 256;

// R = I + 2 (E + F) in place of F (float32), and its bf16 copy when `act` is
// given. Flat over nblocks * b * b floats in float4 steps; b % 4 == 0, so a
// float4 never crosses a row.
__global__ void __launch_bounds__(kNT)
cnp_finish_kernel(const float* __restrict__ E, float* __restrict__ RF, bf16_t* __restrict__ act,
                  int64_t n4, int b) {
  const int64_t bb = (int64_t)b * b;
  for (int64_t q = (int64_t)blockIdx.x * kNT + threadIdx.x; q < n4; q += (int64_t)gridDim.x * kNT) {
    const int64_t e0 = 4 * q;
    const float4 e = *reinterpret_cast<const float4*>(E + e0);
    const float4 f = *reinterpret_cast<const float4*>(RF + e0);
    const int64_t p = e0 % bb;
    const int i = (int)(p / b), j = (int)(p - (int64_t)i * b);
    float r[4] = {2.0f * (e.x + f.x), 2.0f * (e.y + f.y), 2.0f * (e.z + f.z), 2.0f * (e.w + f.w)};
#pragma unroll
    for (int t = 0; t < 4; ++t) r[t] += (i == j + t) ? 1.0f : 0.0f;
    *reinterpret_cast<float4*>(RF + e0) = make_float4(r[0], r[1], r[2], r[3]);
    if (act) {
      union { uint2 u; bf16_t h[4]; } o;
#pragma unroll
      for (int t = 0; t < 4; ++t) o.h[t] = f32_to_bf16(r[t]);
      *reinterpret_cast<uint2*>(act + e0) = o.u;
    }
  }
}

// Four consecutive elements (4 q .. 4 q + 3) as floats, and back.
__device__ __forceinline__ float4 ld4(const float* p, int64_t q) {
  return reinterpret_cast<const float4*>(p)[q];
}
__device__ __forceinline__ float4 ld4(const bf16_t* p, int64_t q) {
  union { uint2 u; bf16_t h[4]; } v;
  v.u = reinterpret_cast<const uint2*>(p)[q];
  return make_float4(bf16_to_f32(v.h[0]), bf16_to_f32(v.h[1]), bf16_to_f32(v.h[2]),
                     bf16_to_f32(v.h[3]));
}
__device__ __forceinline__ void st4(float* p, int64_t q, float4 x) {
  reinterpret_cast<float4*>(p)[q] = x;
}
__device__ __forceinline__ void st4(bf16_t* p, int64_t q, float4 x) {
  union { uint2 u; bf16_t h[4]; } v;
  v.h[0] = f32_to_bf16(x.x); v.h[1] = f32_to_bf16(x.y);
  v.h[2] = f32_to_bf16(x.z); v.h[3] = f32_to_bf16(x.w);
  reinterpret_cast<uint2*>(p)[q] = v.u;
}

// C = A - B (B NULL: C = A, a conversion), flat in steps of 4 elements; the
// difference in float32, rounded once to C's type. A second segment (A2,
// B2, C2, m4 steps) may follow in the same launch: steps n4 .. n4 + m4 - 1.
template <typename TA, typename TB, typename TC>
__global__ void __launch_bounds__(kNT)
sub_kernel(const TA* __restrict__ A, const TB* __restrict__ B, TC* __restrict__ C, int64_t n4,
           const TA* __restrict__ A2, const TB* __restrict__ B2, TC* __restrict__ C2,
           int64_t m4) {
  for (int64_t q = (int64_t)blockIdx.x * kNT + threadIdx.x; q < n4 + m4;
       q += (int64_t)gridDim.x * kNT) {
    const bool two = q >= n4;
    const TA* a_ = two ? A2 : A;
    const TB* b_ = two ? B2 : B;
    TC* c_ = two ? C2 : C;
    const int64_t r = two ? q - n4 : q;
    float4 a = ld4(a_, r);
    if (b_) {
      const float4 c = ld4(b_, r);
      a = make_float4(a.x - c.x, a.y - c.y, a.z - c.z, a.w - c.w);
    }
    st4(c_, r, a);
  }
}

// W = S + S^T with S = A + B, per b x b block, in float32, rounded once to
// W's type. grid (tiles of 32 x 32, nblocks): each workgroup writes tile
// (TI, TJ) from tiles (TI, TJ) and (TJ, TI) of S, the second transposed
// through LDS.
template <typename TIn, typename TOut>
__global__ void __launch_bounds__(kNT)
sym_sum_kernel(const TIn* __restrict__ A, const TIn* __restrict__ B, TOut* __restrict__ W,
               int b, int nb1, const TIn* __restrict__ A2, const TIn* __restrict__ B2,
               TOut* __restrict__ W2) {
  // blocks y < nb1 of (A, B, W), then those of the second set
  __shared__ float s1[32][33], s2[32][33];
  const int ntile = (b + 31) / 32;
  const int TI = blockIdx.x / ntile, TJ = blockIdx.x - TI * ntile;
  const bool two = (int)blockIdx.y >= nb1;
  if (two) {
    A = A2;
    B = B2;
    W = W2;
  }
  const int64_t base = (int64_t)(two ? (int)blockIdx.y - nb1 : (int)blockIdx.y) * b * b;
  const int tx = threadIdx.x & 31, ty0 = threadIdx.x >> 5;
  for (int ty = ty0; ty < 32; ty += 8) {
    const int i = TI * 32 + ty, j = TJ * 32 + tx;
    float v = 0.0f;
    if (i < b && j < b)
      v = ElemTraits<TIn>::to_f32(A[base + (int64_t)i * b + j]) +
          ElemTraits<TIn>::to_f32(B[base + (int64_t)i * b + j]);
    s1[ty][tx] = v;
    const int it = TJ * 32 + ty, jt = TI * 32 + tx;
    float w = 0.0f;
    if (it < b && jt < b)
      w = ElemTraits<TIn>::to_f32(A[base + (int64_t)it * b + jt]) +
          ElemTraits<TIn>::to_f32(B[base + (int64_t)it * b + jt]);
    s2[ty][tx] = w;
  }
  __syncthreads();
  for (int ty = ty0; ty < 32; ty += 8) {
    const int i = TI * 32 + ty, j = TJ * 32 + tx;
    if (i < b && j < b) store_as<TOut>(W + base + (int64_t)i * b + j, s1[ty][tx] + s2[tx][ty]);
  }
}

int flat_grid(int64_t n4) {
  const int64_t g = (n4 + kNT - 1) / kNT;
  return (int)std::min<int64_t>(g, 4096);
}

}  // namespace

hipError_t launch_cnp_finish(const float* E, float* RF, void* act_bf16, int64_t nblocks, int b,
                             hipStream_t stream) {
  const int64_t n4 = nblocks * b * b / 4;
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(cnp_finish_kernel, dim3(flat_grid(n4)), dim3(kNT), 0, stream, E, RF,
                     static_cast<bf16_t*>(act_bf16), n4, b);
  return hipGetLastError();
}

hipError_t launch_sub(const float* A, const float* B, float* C, int64_t n, hipStream_t stream) {
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL((sub_kernel<float, float, float>), dim3(flat_grid(n4)), dim3(kNT), 0, stream,
                     A, B, C, n4, nullptr, nullptr, nullptr, (int64_t)0);
  return hipGetLastError();
}

hipError_t launch_sub_to_bf16(DType ta, const void* A, const float* B, void* C, int64_t n,
                              const void* A2, const float* B2, void* C2, int64_t n2,
                              hipStream_t stream) {
  if (n % 4 != 0 || n2 % 4 != 0 || n2 < 0) return hipErrorInvalidValue;
  const int64_t n4 = n / 4, m4 = n2 / 4;
  if (n4 + m4 == 0) return hipSuccess;
  if (ta == DType::BF16)
    hipLaunchKernelGGL((sub_kernel<bf16_t, float, bf16_t>), dim3(flat_grid(n4 + m4)), dim3(kNT), 0,
                       stream, static_cast<const bf16_t*>(A), B, static_cast<bf16_t*>(C), n4,
                       static_cast<const bf16_t*>(A2), B2, static_cast<bf16_t*>(C2), m4);
  else
    hipLaunchKernelGGL((sub_kernel<float, float, bf16_t>), dim3(flat_grid(n4 + m4)), dim3(kNT), 0,
                       stream, static_cast<const float*>(A), B, static_cast<bf16_t*>(C), n4,
                       static_cast<const float*>(A2), B2, static_cast<bf16_t*>(C2), m4);
  return hipGetLastError();
}

hipError_t launch_sym_sum(const float* A, const float* B, float* W, int64_t nblocks, int b,
                          hipStream_t stream) {
  if (nblocks == 0) return hipSuccess;
  const int nt = (b + 31) / 32;
  hipLaunchKernelGGL((sym_sum_kernel<float, float>), dim3(nt * nt, (int)nblocks), dim3(kNT), 0,
                     stream, A, B, W, b, (int)nblocks, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_sym_sum_bf16(const void* A, const void* B, void* W, int64_t nblocks,
                               const void* A2, const void* B2, void* W2, int64_t nblocks2, int b,
                               hipStream_t stream) {
  if (nblocks + nblocks2 == 0) return hipSuccess;
  const int nt = (b + 31) / 32;
  hipLaunchKernelGGL((sym_sum_kernel<bf16_t, bf16_t>), dim3(nt * nt, (int)(nblocks + nblocks2)),
                     dim3(kNT), 0, stream, static_cast<const bf16_t*>(A),
                     static_cast<const bf16_t*>(B), static_cast<bf16_t*>(W), b, (int)nblocks,
                     static_cast<const bf16_t*>(A2), static_cast<const bf16_t*>(B2),
                     static_cast<bf16_t*>(W2));
  return hipGetLastError();
}

}  // namespace poetx
