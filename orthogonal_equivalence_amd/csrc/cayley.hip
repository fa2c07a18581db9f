// Exact Cayley map of packed skew generators, and the small kernels of the
// Cayley backward.
//
// Method: skew-symmetric generators Q = -Q^T stored as the strict upper
// triangle (gist.science technical summary of "POET-X: Memory-efficient LLM
// Training by Scaling Orthogonal Transformation", section 2 Methodik,
// Cayley-Neumann parameterisation item). The map used here is the exact
// Cayley map R = (I + Q)(I - Q)^-1 = 2 (I - Q)^-1 - I.
//
// (I - Q)^-1 is formed by blocked Gauss-Jordan elimination without pivoting,
// in place in the float32 output buffer: I - Q has symmetric part I, which
// is positive definite, so every leading pivot block (a Schur complement of
// I - Q) again has a positive definite symmetric part and is invertible.
// Each panel of width pw is one pair of launches over all blocks at once:
//   prep:   D = A[p][p] is inverted in LDS by scalar Gauss-Jordan; the
//           workgroup for column tile J writes Dinv A[p][J] (Dinv itself for
//           J = p) to a row-panel buffer and copies A[J][p] to a column-panel
//           buffer;
//   update: every tile (I, J) becomes rowpanel[J] (I = p) or
//           A[I][J] - colpanel[I] rowpanel[J] (A[I][p] taken as zero).
// The last update writes R = 2 B - I and the activation-type copy.
#include "common.h"
#include "kernels.h"

namespace poetx {
namespace {

constexpr int kPW = 64;  // maximum panel width
constexpr int kNT = 256; // threads per workgroup

__device__ __forceinline__ int64_t packed_index(int b, int i, int j) {
  // position of (i, j), i < j, in the row-major strict upper triangle
  return (int64_t)i * (2 * b - i - 1) / 2 + (j - i - 1);
}

// A = I - Q for every block; the last block's rows/columns >= last_valid are
// identity (generator entries there are ignored).
__global__ void __launch_bounds__(kNT)
expand_kernel(const float* __restrict__ theta, int64_t nblocks, int b, int last_valid,
              float* __restrict__ A) {
  const int64_t bb = (int64_t)b * b;
  const int64_t total = nblocks * bb;
  const int64_t tri = (int64_t)b * (b - 1) / 2;
  for (int64_t idx = blockIdx.x * (int64_t)kNT + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * kNT) {
    const int64_t blk = idx / bb;
    const int ij = (int)(idx - blk * bb);
    const int i = ij / b, j = ij - (ij / b) * b;
    const int r = (blk == nblocks - 1) ? last_valid : b;
    float v;
    if (i == j) v = 1.0f;
    else if (i >= r || j >= r) v = 0.0f;
    else if (i < j) v = -theta[blk * tri + packed_index(b, i, j)];
    else v = theta[blk * tri + packed_index(b, j, i)];
    A[idx] = v;
  }
}

// Gauss-Jordan inverse of the pw x pw matrix in sD (row stride kPW + 1),
// in place, no pivoting.
__device__ void gj_invert(float (*sD)[kPW + 1], float* rowk, float* colk, int pw) {
  const int tid = threadIdx.x;
  for (int k = 0; k < pw; ++k) {
    __syncthreads();
    const float pinv = 1.0f / sD[k][k];
    for (int t = tid; t < pw; t += kNT) {
      rowk[t] = (t == k) ? pinv : sD[k][t] * pinv;
      colk[t] = (t == k) ? 0.0f : sD[t][k];
    }
    __syncthreads();
    for (int e = tid; e < pw * pw; e += kNT) {
      const int i = e / pw, j = e - (e / pw) * pw;
      if (i == k) sD[i][j] = rowk[j];
      else sD[i][j] = (j == k ? 0.0f : sD[i][j]) - colk[i] * rowk[j];
    }
  }
  __syncthreads();
}

// grid (b / pw column tiles, nblocks)
__global__ void __launch_bounds__(kNT)
panel_prep_kernel(const float* __restrict__ A, int b, int pw, int p,
                  float* __restrict__ rowbuf, float* __restrict__ colbuf) {
  __shared__ float sD[kPW][kPW + 1];
  __shared__ float sX[kPW][kPW + 1];
  __shared__ float rowk[kPW], colk[kPW];
  const int tid = threadIdx.x;
  const int J = blockIdx.x;
  const int64_t blk = blockIdx.y;
  const float* Ab = A + blk * (int64_t)b * b;
  const int p0 = p * pw, j0 = J * pw;

  for (int e = tid; e < pw * pw; e += kNT) {
    const int i = e / pw, j = e - (e / pw) * pw;
    sD[i][j] = Ab[(int64_t)(p0 + i) * b + p0 + j];
    // column panel rows of tile J (unused for J == p)
    colbuf[(blk * b + j0 + i) * pw + j] = Ab[(int64_t)(j0 + i) * b + p0 + j];
    if (J != p) sX[i][j] = Ab[(int64_t)(p0 + i) * b + j0 + j];
  }
  gj_invert(sD, rowk, colk, pw);

  float* rb = rowbuf + blk * (int64_t)pw * b;
  for (int e = tid; e < pw * pw; e += kNT) {
    const int i = e / pw, j = e - (e / pw) * pw;
    float v;
    if (J == p) {
      v = sD[i][j];
    } else {
      v = 0.0f;
      for (int c = 0; c < pw; ++c) v = fmaf(sD[i][c], sX[c][j], v);
    }
    rb[(int64_t)i * b + j0 + j] = v;
  }
}

// grid (nt * nt tiles, nblocks). When `final` is set the tile is written as
// R = 2 B - I to A (the float32 output) and to `act_out` (bf16), if given.
__global__ void __launch_bounds__(kNT)
panel_update_kernel(float* __restrict__ A, int b, int pw, int p,
                    const float* __restrict__ rowbuf, const float* __restrict__ colbuf,
                    int final, bf16_t* __restrict__ act_out) {
  __shared__ float sC[kPW][kPW + 1];
  __shared__ float sR[kPW][kPW + 1];
  const int tid = threadIdx.x;
  const int nt = b / pw;
  const int I = blockIdx.x / nt, J = blockIdx.x - (blockIdx.x / nt) * nt;
  const int64_t blk = blockIdx.y;
  float* Ab = A + blk * (int64_t)b * b;
  const float* rb = rowbuf + blk * (int64_t)pw * b;
  const float* cb = colbuf + blk * (int64_t)b * pw;
  const int i0 = I * pw, j0 = J * pw;

  for (int e = tid; e < pw * pw; e += kNT) {
    const int i = e / pw, j = e - (e / pw) * pw;
    sR[i][j] = rb[(int64_t)i * b + j0 + j];
    sC[i][j] = (I == p) ? 0.0f : cb[(int64_t)(i0 + i) * pw + j];
  }
  __syncthreads();

  // thread (ty, tx) of a 16 x 16 grid owns rows ty + 16 a and columns
  // tx + 16 c, a, c < 4
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = ty + 16 * a, j = tx + 16 * c;
      float v = 0.0f;
      if (i < pw && j < pw) {
        if (I == p) v = sR[i][j];
        else if (J != p) v = Ab[(int64_t)(i0 + i) * b + j0 + j];
      }
      acc[a][c] = v;
    }
  if (I != p) {
    for (int k = 0; k < pw; ++k) {
      float cv[4], rv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) cv[a] = (ty + 16 * a < pw) ? sC[ty + 16 * a][k] : 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) rv[c] = (tx + 16 * c < pw) ? sR[k][tx + 16 * c] : 0.0f;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = fmaf(-cv[a], rv[c], acc[a][c]);
    }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = ty + 16 * a, j = tx + 16 * c;
      if (i < pw && j < pw) {
        const int64_t off = (int64_t)(i0 + i) * b + j0 + j;
        float v = acc[a][c];
        if (final) {
          v = 2.0f * v - ((i0 + i) == (j0 + j) ? 1.0f : 0.0f);
          if (act_out) act_out[blk * (int64_t)b * b + off] = f32_to_bf16(v);
        }
        Ab[off] = v;
      }
    }
}

__global__ void __launch_bounds__(kNT)
split_reduce_kernel(const float* __restrict__ part, int nsplit, int64_t nblocks, int b,
                    int last_valid, float* __restrict__ G) {
  const int64_t bb = (int64_t)b * b;
  const int64_t total = nblocks * bb;
  for (int64_t idx = blockIdx.x * (int64_t)kNT + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * kNT) {
    const int64_t blk = idx / bb;
    const int ij = (int)(idx - blk * bb);
    const int i = ij / b, j = ij - (ij / b) * b;
    float v = 0.0f;
    if (blk != nblocks - 1 || (i < last_valid && j < last_valid)) {
      for (int s = 0; s < nsplit; ++s) v += part[(int64_t)s * total + idx];
    }
    G[idx] = v;
  }
}

__global__ void __launch_bounds__(kNT)
pack_skew_grad_kernel(const float* __restrict__ M, int64_t nblocks, int b, int last_valid,
                      float* __restrict__ g) {
  const int64_t bb = (int64_t)b * b;
  const int64_t total = nblocks * bb;
  const int64_t tri = (int64_t)b * (b - 1) / 2;
  for (int64_t idx = blockIdx.x * (int64_t)kNT + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * kNT) {
    const int64_t blk = idx / bb;
    const int ij = (int)(idx - blk * bb);
    const int i = ij / b, j = ij - (ij / b) * b;
    if (i >= j) continue;
    const int r = (blk == nblocks - 1) ? last_valid : b;
    const float* Mb = M + blk * bb;
    const float v = (j < r) ? Mb[(int64_t)i * b + j] - Mb[(int64_t)j * b + i] : 0.0f;
    g[blk * tri + packed_index(b, i, j)] = v;
  }
}

inline unsigned grid_for(int64_t total) {
  int64_t g = (total + kNT - 1) / kNT;
  if (g > 65536) g = 65536;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

int cayley_panel_width(int b) {
  if (b <= kPW) return b;
  int pw = kPW;
  while (b % pw) pw >>= 1;
  return pw;
}

size_t cayley_workspace_floats(int64_t nblocks, int b) {
  const int pw = cayley_panel_width(b);
  return 2 * (size_t)nblocks * (size_t)pw * (size_t)b;
}

hipError_t launch_cayley_build(const float* theta, int64_t nblocks, int b, int last_valid,
                               float* blocks_f32, void* blocks_act, DType act, float* ws,
                               hipStream_t stream) {
  const int pw = cayley_panel_width(b);
  const int nt = b / pw;
  float* rowbuf = ws;
  float* colbuf = ws + (size_t)nblocks * pw * b;
  bf16_t* act_out = (act == DType::BF16) ? static_cast<bf16_t*>(blocks_act) : nullptr;
  hipLaunchKernelGGL(expand_kernel, dim3(grid_for(nblocks * (int64_t)b * b)), dim3(kNT), 0, stream,
                     theta, nblocks, b, last_valid, blocks_f32);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int p = 0; p < nt; ++p) {
    hipLaunchKernelGGL(panel_prep_kernel, dim3(nt, (unsigned)nblocks), dim3(kNT), 0, stream,
                       blocks_f32, b, pw, p, rowbuf, colbuf);
    hipLaunchKernelGGL(panel_update_kernel, dim3(nt * nt, (unsigned)nblocks), dim3(kNT), 0, stream,
                       blocks_f32, b, pw, p, rowbuf, colbuf, (int)(p == nt - 1), act_out);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_split_reduce(const float* part, int nsplit, int64_t nblocks, int b,
                               int last_valid, float* G, hipStream_t stream) {
  hipLaunchKernelGGL(split_reduce_kernel, dim3(grid_for(nblocks * (int64_t)b * b)), dim3(kNT), 0,
                     stream, part, nsplit, nblocks, b, last_valid, G);
  return hipGetLastError();
}

hipError_t launch_pack_skew_grad(const float* M, int64_t nblocks, int b, int last_valid,
                                 float* g_theta, hipStream_t stream) {
  hipLaunchKernelGGL(pack_skew_grad_kernel, dim3(grid_for(nblocks * (int64_t)b * b)), dim3(kNT), 0,
                     stream, M, nblocks, b, last_valid, g_theta);
  return hipGetLastError();
}

}  // namespace poetx
