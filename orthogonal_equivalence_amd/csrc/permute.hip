// Block-mixing permutations applied as index maps on token-major data.
//
// Method (gist.science technical summary of "POET-X: Memory-efficient LLM
// Training by Scaling Orthogonal Transformation", section 2 Methodik,
// permutation item): the permutations that mix the blocks of R and P are not
// built as matrices; index maps (bijections) are applied to the data
// directly, and the two inner permutations of the forward are folded into
// the weight once.
//
// Column gather: out[r][j] = in[src(r)][perm[j]], src(r) = rowmap[r] or r.
// An index outside [0, d) reads as zero, so a bad map gives wrong values but
// never an out-of-bounds access. A scatter out[r][perm[i]] = in[r][i] is the
// gather by the inverse map, which invert_kernel builds on the device.
//
// MI355X layout: a row of up to 64 KB is first copied into LDS with 16-byte
// coalesced loads; each thread then assembles 16 output bytes from LDS
// (random 2- or 4-byte LDS reads, indices held in registers) and writes them
// with one coalesced 16-byte store. HBM traffic is one read and one write of
// the row. Longer rows take a plain kernel that gathers straight from global
// memory (L2-resident rows).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace poetx {
namespace {

constexpr int kNT = 256;
constexpr int kMaxLdsBytes = 64 * 1024;

template <typename T> struct Vec16;
template <> struct Vec16<bf16_t> { static constexpr int N = 8; };
template <> struct Vec16<float> { static constexpr int N = 4; };

// Persistent over rows: each thread owns the output chunks c = tid + i NT
// (i < CPT) of every row and keeps their indices in registers, so the map is
// read once per workgroup rather than once per row (an int32 map is twice the
// bytes of a bf16 row). Rows go global -> LDS -> gathered registers -> global.
// grid: up to a few workgroups per CU striding over rows; dynamic LDS d * sizeof(T).
template <typename T, int NT, int CPT>
__global__ void __launch_bounds__(NT)
gather_lds_kernel(const T* __restrict__ in, int64_t ld_in, const int32_t* __restrict__ rowmap,
                  int64_t in_rows, int64_t rows, int d, const int32_t* __restrict__ perm,
                  T* __restrict__ out, int64_t ld_out) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  T* row = reinterpret_cast<T*>(smem_raw);
  constexpr int V = Vec16<T>::N;
  const int nvec = d / V;  // d % V == 0 and nvec <= NT * CPT (host checks)
  int idx[CPT][V];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = threadIdx.x + i * NT;
#pragma unroll
    for (int t = 0; t < V; ++t) {
      int p = -1;
      if (c < nvec) p = perm[c * V + t];
      idx[i][t] = ((unsigned)p < (unsigned)d) ? p : -1;
    }
  }
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    int64_t src = r;
    if (rowmap) src = rowmap[r];
    const bool src_ok = src >= 0 && src < in_rows;
    __syncthreads();  // the previous row's LDS reads are done
    if (src_ok) {
      const uint4* s = reinterpret_cast<const uint4*>(in + src * ld_in);
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = threadIdx.x + i * NT;
        if (c < nvec) reinterpret_cast<uint4*>(row)[c] = s[c];
      }
    }
    __syncthreads();
    uint4* o = reinterpret_cast<uint4*>(out + r * ld_out);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = threadIdx.x + i * NT;
      if (c >= nvec) break;
      union { uint4 u; T e[V]; } v;
#pragma unroll
      for (int t = 0; t < V; ++t) v.e[t] = (src_ok && idx[i][t] >= 0) ? row[idx[i][t]] : T(0);
      o[c] = v.u;
    }
  }
}

// the same map without LDS staging, for rows longer than kMaxLdsBytes;
// out must not overlap in. grid (ceil(d / (V kNT)), row chunks)
template <typename T>
__global__ void __launch_bounds__(kNT)
gather_global_kernel(const T* __restrict__ in, int64_t ld_in, const int32_t* __restrict__ rowmap,
                     int64_t in_rows, int64_t rows, int d, const int32_t* __restrict__ perm,
                     T* __restrict__ out, int64_t ld_out) {
  constexpr int V = Vec16<T>::N;
  const int c = blockIdx.x * kNT + threadIdx.x;
  if (c * V >= d) return;
  int idx[V];
#pragma unroll
  for (int t = 0; t < V; ++t) idx[t] = perm[c * V + t];
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    int64_t src = r;
    if (rowmap) src = rowmap[r];
    const bool src_ok = src >= 0 && src < in_rows;
    const T* s = in + src * ld_in;
    union { uint4 u; T e[V]; } v;
#pragma unroll
    for (int t = 0; t < V; ++t)
      v.e[t] = (src_ok && (unsigned)idx[t] < (unsigned)d) ? s[idx[t]] : T(0);
    reinterpret_cast<uint4*>(out + r * ld_out)[c] = v.u;
  }
}

__global__ void __launch_bounds__(kNT)
fill_i32_kernel(int32_t* __restrict__ p, int d, int32_t v) {
  const int i = blockIdx.x * kNT + threadIdx.x;
  if (i < d) p[i] = v;
}

// inv[perm[i]] = i for every in-range entry (run after filling inv with -1)
__global__ void __launch_bounds__(kNT)
invert_kernel(const int32_t* __restrict__ perm, int d, int32_t* __restrict__ inv) {
  const int i = blockIdx.x * kNT + threadIdx.x;
  if (i >= d) return;
  const int p = perm[i];
  if ((unsigned)p < (unsigned)d) inv[p] = i;
}

template <typename T>
hipError_t gather_t(const void* in, int64_t ld_in, const int32_t* rowmap, int64_t in_rows,
                    int64_t rows, int d, const int32_t* perm, void* out, int64_t ld_out,
                    hipStream_t s) {
  constexpr int V = Vec16<T>::N;
  if (rows == 0 || d == 0) return hipSuccess;
  const size_t lds = (size_t)d * sizeof(T);
  const int nvec = d / V;
  if (lds <= (size_t)kMaxLdsBytes && in != out) {
    // about four rows in flight per CU (LDS allowing), each workgroup then
    // streams its share of the rows
    const int per_cu = (int)std::max<size_t>(1, std::min<size_t>(4, (160 * 1024) / std::max<size_t>(lds, 1)));
    const int64_t grid = std::min<int64_t>(rows, (int64_t)256 * per_cu);
    if (nvec <= 256 * 8)
      hipLaunchKernelGGL((gather_lds_kernel<T, 256, 8>), dim3((unsigned)grid), dim3(256), lds, s,
                         static_cast<const T*>(in), ld_in, rowmap, in_rows, rows, d, perm,
                         static_cast<T*>(out), ld_out);
    else
      hipLaunchKernelGGL((gather_lds_kernel<T, 512, 8>), dim3((unsigned)grid), dim3(512), lds, s,
                         static_cast<const T*>(in), ld_in, rowmap, in_rows, rows, d, perm,
                         static_cast<T*>(out), ld_out);
  } else if (in != out) {
    const int gx = (d / V + kNT - 1) / kNT;
    const int64_t gy = std::min<int64_t>(rows, std::max<int64_t>(1, 8192 / gx));
    hipLaunchKernelGGL(gather_global_kernel<T>, dim3(gx, (unsigned)gy), dim3(kNT), 0, s,
                       static_cast<const T*>(in), ld_in, rowmap, in_rows, rows, d, perm,
                       static_cast<T*>(out), ld_out);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather_columns(DType t, const void* in, int64_t ld_in, const int32_t* rowmap,
                                 int64_t in_rows, int64_t rows, int d, const int32_t* perm,
                                 void* out, int64_t ld_out, hipStream_t s) {
  return t == DType::BF16 ? gather_t<bf16_t>(in, ld_in, rowmap, in_rows, rows, d, perm, out, ld_out, s)
                          : gather_t<float>(in, ld_in, rowmap, in_rows, rows, d, perm, out, ld_out, s);
}

hipError_t launch_invert_permutation(const int32_t* perm, int d, int32_t* inv, hipStream_t s) {
  if (d == 0) return hipSuccess;
  const int g = (d + kNT - 1) / kNT;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(g), dim3(kNT), 0, s, inv, d, -1);
  hipLaunchKernelGGL(invert_kernel, dim3(g), dim3(kNT), 0, s, perm, d, inv);
  return hipGetLastError();
}

}  // namespace poetx
