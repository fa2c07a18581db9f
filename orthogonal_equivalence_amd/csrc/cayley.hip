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
// is positive definite, so every pivot block (a Schur complement of I - Q)
// again has a positive definite symmetric part and is invertible. Each panel
// of width pw (<= 64) is one pair of launches over all blocks at once:
//   prep:   D = A[p][p] is inverted in registers (each of 256 threads owns a
//           4 x 4 piece; the pivot row and column go through LDS, one barrier
//           per elimination step); the workgroup for column tile J writes
//           W_J = Dinv A[p][J] (Dinv itself for J = p, an fp32 MFMA product
//           otherwise) to a row-panel buffer and copies A[J][p] to a
//           column-panel buffer;
//   update: every tile (I, J) becomes W_J (I = p) or
//           A[I][J] - colpanel[I] W_J (A[I][p] taken as zero), on MFMA.
// The last update writes R = 2 B - I and the activation-type copy.
#include "common.h"
#include "kernels.h"

namespace poetx {
namespace {

constexpr int kPW = 64;   // maximum panel width
constexpr int kNT = 256;  // threads per workgroup (a 16 x 16 grid of 4 x 4 pieces)
constexpr int kLdA = 68;  // LDS row stride of a 64 x 64 MFMA A operand ([m][k])
constexpr int kLdB = 80;  // LDS row stride of a 64 x 64 MFMA B operand ([k][n])

__device__ __forceinline__ int packed_index(int b, int i, int j) {
  // position of (i, j), i < j, in the row-major strict upper triangle
  return i * (2 * b - i - 1) / 2 + (j - i - 1);
}

// A = I - Q for every block; the last block's rows/columns >= last_valid
// are identity. grid (tiles of 32 x 32, nblocks). A tile below the diagonal
// reads its generators from the mirrored tile above it (coalesced along the
// packed rows) and transposes through LDS.
__global__ void __launch_bounds__(kNT)
expand_kernel(const float* __restrict__ theta, int nblocks, int b, int last_valid,
              float* __restrict__ A) {
  __shared__ float t[32][33];
  const int ntile = (b + 31) / 32;
  const int TI = blockIdx.x / ntile, TJ = blockIdx.x - (blockIdx.x / ntile) * ntile;
  const int blk = blockIdx.y;
  const int r = (blk == nblocks - 1) ? last_valid : b;
  const float* th = theta + (int64_t)blk * (b * (b - 1) / 2);
  float* Ab = A + (int64_t)blk * b * b;
  const int tx = threadIdx.x & 31, ty0 = threadIdx.x >> 5;  // 8 rows per pass
  const bool lower = TI > TJ;
  // read the upper-triangle tile (lower ? (TJ, TI) : (TI, TJ)) row by row
  const int ui = lower ? TJ : TI, uj = lower ? TI : TJ;
  for (int ty = ty0; ty < 32; ty += 8) {
    const int i = ui * 32 + ty, j = uj * 32 + tx;
    float q = 0.0f;  // Q[i][j]
    if (i < j && j < b && i < r && j < r) q = th[packed_index(b, i, j)];
    t[ty][tx] = q;
  }
  __syncthreads();
  for (int ty = ty0; ty < 32; ty += 8) {
    const int i = TI * 32 + ty, j = TJ * 32 + tx;
    if (i >= b || j >= b) continue;
    float v;
    if (i == j) v = 1.0f;
    else if (i > j) v = t[tx][ty];  // A[i][j] = -Q[i][j] = Q[j][i]
    else v = -t[ty][tx];
    Ab[(int64_t)i * b + j] = v;
  }
}

// Reciprocal: hardware estimate refined by one Newton step (error ~1 ulp).
__device__ __forceinline__ float recip(float x) {
  float r = __builtin_amdgcn_rcpf(x);
  return fmaf(r, fmaf(-x, r, 1.0f), r);
}

// One elimination step k = 4 k4 + KK of gj_invert_regs (KK compile-time, so
// every register index is static).
template <int KK>
__device__ __forceinline__ void gj_step(float a[4][4], int k4, float* rowb, float* colb) {
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int k = 4 * k4 + KK;
  const bool own_row = ty == k4, own_col = tx == k4;
  if (own_row)
    *reinterpret_cast<float4*>(&rowb[4 * tx]) = make_float4(a[KK][0], a[KK][1], a[KK][2], a[KK][3]);
  if (own_col)
    *reinterpret_cast<float4*>(&colb[4 * ty]) = make_float4(a[0][KK], a[1][KK], a[2][KK], a[3][KK]);
  __syncthreads();
  const float pinv = recip(rowb[k]);
  const float4 r = *reinterpret_cast<const float4*>(&rowb[4 * tx]);
  const float4 c = *reinterpret_cast<const float4*>(&colb[4 * ty]);
  const float rs[4] = {r.x * pinv, r.y * pinv, r.z * pinv, r.w * pinv};
  const float cv[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) a[ii][jj] = fmaf(-cv[ii], rs[jj], a[ii][jj]);
  if (own_col) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) a[ii][KK] = -cv[ii] * pinv;
  }
  if (own_row) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) a[KK][jj] = rs[jj];
    if (own_col) a[KK][KK] = pinv;
  }
}

// In-place Gauss-Jordan inverse of the leading pw x pw part of a 64 x 64
// matrix distributed as 4 x 4 register pieces (thread (ty, tx) owns rows
// 4ty.., columns 4tx..); entries outside pw x pw must hold the identity.
// Step k: the owners of row k and column k publish them through LDS (double
// buffered, so one barrier per step); every thread applies the rank-1 update
// a -= c r / a_kk to its piece, then the owners of row k and column k
// overwrite them with r / a_kk and -c / a_kk (and a_kk with 1 / a_kk).
__device__ __forceinline__ void gj_invert_regs(float a[4][4], int pw, float (*rowb)[kPW],
                                               float (*colb)[kPW]) {
  for (int k4 = 0; 4 * k4 < pw; ++k4) {
    gj_step<0>(a, k4, rowb[0], colb[0]);
    if (4 * k4 + 1 < pw) gj_step<1>(a, k4, rowb[1], colb[1]);
    if (4 * k4 + 2 < pw) gj_step<2>(a, k4, rowb[0], colb[0]);
    if (4 * k4 + 3 < pw) gj_step<3>(a, k4, rowb[1], colb[1]);
  }
  __syncthreads();
}

// acc (this wave's 32 x 32 quadrant of a 64 x 64 product) += sA sB, with sA
// [64][kLdA] (A[m][k]) and sB [64][kLdB] (B[k][n]) in LDS; fp32 MFMA.
__device__ __forceinline__ void mma64(const float* sA, const float* sB, floatx4 acc[2][2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = (wave >> 1) * 32, c0 = (wave & 1) * 32;
#pragma unroll 4
  for (int k0 = 0; k0 < kPW; k0 += 4) {
    const int k = k0 + (lane >> 4);
    const float a0 = sA[(r0 + (lane & 15)) * kLdA + k];
    const float a1 = sA[(r0 + 16 + (lane & 15)) * kLdA + k];
    const float b0 = sB[k * kLdB + c0 + (lane & 15)];
    const float b1 = sB[k * kLdB + c0 + 16 + (lane & 15)];
    acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b0, acc[0][0], 0, 0, 0);
    acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b1, acc[0][1], 0, 0, 0);
    acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b0, acc[1][0], 0, 0, 0);
    acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b1, acc[1][1], 0, 0, 0);
  }
}

// Row / column of accumulator element e of mma64's output for this lane.
__device__ __forceinline__ int mma_row(int mi, int e) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave >> 1) * 32 + mi * 16 + 4 * (lane >> 4) + e;
}
__device__ __forceinline__ int mma_col(int ni) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave & 1) * 32 + ni * 16 + (lane & 15);
}

// grid (b / pw column tiles, nblocks)
__global__ void __launch_bounds__(kNT)
panel_prep_kernel(const float* __restrict__ A, int b, int pw, int p,
                  float* __restrict__ rowbuf, float* __restrict__ colbuf) {
  __shared__ __attribute__((aligned(16))) float sD[kPW * kLdA];
  __shared__ __attribute__((aligned(16))) float sX[kPW * kLdB];
  __shared__ __attribute__((aligned(16))) float rowb[2][kPW];
  __shared__ __attribute__((aligned(16))) float colb[2][kPW];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int J = blockIdx.x;
  const int64_t blk = blockIdx.y;
  const float* Ab = A + blk * (int64_t)b * b;
  const int p0 = p * pw, j0 = J * pw;

  float a[4][4];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int gi = 4 * ty + ii, gj = 4 * tx + jj;
      const bool in = gi < pw && gj < pw;
      a[ii][jj] = in ? Ab[(int64_t)(p0 + gi) * b + p0 + gj] : (gi == gj ? 1.0f : 0.0f);
      if (in) colbuf[(blk * b + j0 + gi) * pw + gj] = Ab[(int64_t)(j0 + gi) * b + p0 + gj];
      if (J != p) sX[gi * kLdB + gj] = in ? Ab[(int64_t)(p0 + gi) * b + j0 + gj] : 0.0f;
    }
  gj_invert_regs(a, pw, rowb, colb);

  float* rb = rowbuf + blk * (int64_t)pw * b;
  if (J == p) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int gi = 4 * ty + ii, gj = 4 * tx + jj;
        if (gi < pw && gj < pw) rb[(int64_t)gi * b + p0 + gj] = a[ii][jj];
      }
    return;
  }
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) sD[(4 * ty + ii) * kLdA + 4 * tx + jj] = a[ii][jj];
  __syncthreads();
  floatx4 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = floatx4{0.f, 0.f, 0.f, 0.f};
  mma64(sD, sX, acc);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int gi = mma_row(mi, e), gj = mma_col(ni);
        if (gi < pw && gj < pw) rb[(int64_t)gi * b + j0 + gj] = acc[mi][ni][e];
      }
}

// grid (nt * nt tiles, nblocks). When `final` is set the tile is written as
// R = 2 B - I to A (the float32 output) and to `act_out` (bf16), if given.
__global__ void __launch_bounds__(kNT)
panel_update_kernel(float* __restrict__ A, int b, int pw, int p,
                    const float* __restrict__ rowbuf, const float* __restrict__ colbuf,
                    int final, bf16_t* __restrict__ act_out) {
  __shared__ __attribute__((aligned(16))) float sC[kPW * kLdA];
  __shared__ __attribute__((aligned(16))) float sW[kPW * kLdB];
  const int tid = threadIdx.x;
  const int nt = b / pw;
  const int I = blockIdx.x / nt, J = blockIdx.x - (blockIdx.x / nt) * nt;
  const int64_t blk = blockIdx.y;
  float* Ab = A + blk * (int64_t)b * b;
  const float* rb = rowbuf + blk * (int64_t)pw * b;
  const float* cb = colbuf + blk * (int64_t)b * pw;
  const int i0 = I * pw, j0 = J * pw;

  auto emit = [&](int gi, int gj, float v) {
    const int64_t off = (int64_t)(i0 + gi) * b + j0 + gj;
    if (final) {
      v = 2.0f * v - ((i0 + gi) == (j0 + gj) ? 1.0f : 0.0f);
      if (act_out) act_out[blk * (int64_t)b * b + off] = f32_to_bf16(v);
    }
    Ab[off] = v;
  };

  if (I == p) {
    for (int e = tid; e < pw * pw; e += kNT) {
      const int gi = e / pw, gj = e - (e / pw) * pw;
      emit(gi, gj, rb[(int64_t)gi * b + j0 + gj]);
    }
    return;
  }
  {
    // each thread stages a 4 x 4 piece of C (colpanel rows I) and W (rowpanel
    // columns J); pw is a power of two >= 4 here or the whole block (b <= 64)
    const int ty = tid >> 4, tx = tid & 15;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int gi = 4 * ty + ii, gj = 4 * tx;
      float4 c = make_float4(0.f, 0.f, 0.f, 0.f), w = c;
      if (gi < pw && gj < pw) {
        if ((pw & 3) == 0) {
          c = *reinterpret_cast<const float4*>(cb + (int64_t)(i0 + gi) * pw + gj);
          w = *reinterpret_cast<const float4*>(rb + (int64_t)gi * b + j0 + gj);
        } else {
          float ce[4] = {0.f, 0.f, 0.f, 0.f}, we[4] = {0.f, 0.f, 0.f, 0.f};
          for (int t = 0; t < 4 && gj + t < pw; ++t) {
            ce[t] = cb[(int64_t)(i0 + gi) * pw + gj + t];
            we[t] = rb[(int64_t)gi * b + j0 + gj + t];
          }
          c = make_float4(ce[0], ce[1], ce[2], ce[3]);
          w = make_float4(we[0], we[1], we[2], we[3]);
        }
      }
      *reinterpret_cast<float4*>(&sC[gi * kLdA + gj]) = c;
      *reinterpret_cast<float4*>(&sW[gi * kLdB + gj]) = w;
    }
  }
  // the tile's current values, all loaded before any store (the stores go to
  // the same buffer, so the compiler could not move later loads above them)
  float base[2][2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int gi = mma_row(mi, e), gj = mma_col(ni);
        base[mi][ni][e] = (J != p && gi < pw && gj < pw) ? Ab[(int64_t)(i0 + gi) * b + j0 + gj] : 0.0f;
      }
  __syncthreads();
  floatx4 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = floatx4{0.f, 0.f, 0.f, 0.f};
  mma64(sC, sW, acc);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int gi = mma_row(mi, e), gj = mma_col(ni);
        if (gi < pw && gj < pw) emit(gi, gj, base[mi][ni][e] - acc[mi][ni][e]);
      }
}

// grid (ceil(b*b / (4 kNT)), nblocks); b*b is a multiple of 4
template <typename TOut>
__global__ void __launch_bounds__(kNT)
split_reduce_kernel(const float* __restrict__ part, int nsplit, int nblocks, int b,
                    int last_valid, TOut* __restrict__ G) {
  const int q = blockIdx.x * kNT + threadIdx.x;  // float4 index within the block
  const int bb = b * b;
  if (4 * q >= bb) return;
  const int blk = blockIdx.y;
  const int64_t total = (int64_t)nblocks * bb;
  const int64_t off = (int64_t)blk * bb + 4 * q;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < nsplit; ++s) {
    const float4 t = *reinterpret_cast<const float4*>(part + (int64_t)s * total + off);
    v.x += t.x; v.y += t.y; v.z += t.z; v.w += t.w;
  }
  float e[4] = {v.x, v.y, v.z, v.w};
  if (blk == nblocks - 1 && last_valid < b) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int ij = 4 * q + t, i = ij / b, j = ij - (ij / b) * b;
      if (i >= last_valid || j >= last_valid) e[t] = 0.0f;
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) store_as<TOut>(G + off + t, e[t]);
}

// grid (ceil(b*b / kNT), nblocks)
// g_theta(i, j) = sign ((M + c S)[i][j] - (M + c S)[j][i]), S optional (bf16)
__global__ void __launch_bounds__(kNT)
pack_skew_grad_kernel(const float* __restrict__ M, const bf16_t* __restrict__ S, float c, int nblocks,
                      int b, int last_valid, float sign, float* __restrict__ g) {
  const int ij = blockIdx.x * kNT + threadIdx.x;
  if (ij >= b * b) return;
  const int i = ij / b, j = ij - (ij / b) * b;
  if (i >= j) return;
  const int blk = blockIdx.y;
  const int r = (blk == nblocks - 1) ? last_valid : b;
  const int64_t base = (int64_t)blk * b * b;
  const int64_t a = base + (int64_t)i * b + j, t = base + (int64_t)j * b + i;
  float v = 0.0f;
  if (j < r) {
    v = M[a] - M[t];
    if (S) v += c * (bf16_to_f32(S[a]) - bf16_to_f32(S[t]));
    v *= sign;
  }
  g[(int64_t)blk * (b * (b - 1) / 2) + packed_index(b, i, j)] = v;
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
  const int nb = (int)nblocks;
  float* rowbuf = ws;
  float* colbuf = ws + (size_t)nblocks * pw * b;
  bf16_t* act_out = (act == DType::BF16) ? static_cast<bf16_t*>(blocks_act) : nullptr;
  const int et = (b + 31) / 32;
  hipLaunchKernelGGL(expand_kernel, dim3(et * et, nb), dim3(kNT), 0, stream, theta, nb, b,
                     last_valid, blocks_f32);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int p = 0; p < nt; ++p) {
    hipLaunchKernelGGL(panel_prep_kernel, dim3(nt, nb), dim3(kNT), 0, stream, blocks_f32, b, pw, p,
                       rowbuf, colbuf);
    hipLaunchKernelGGL(panel_update_kernel, dim3(nt * nt, nb), dim3(kNT), 0, stream, blocks_f32, b,
                       pw, p, rowbuf, colbuf, (int)(p == nt - 1), act_out);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_split_reduce(const float* part, int nsplit, int64_t nblocks, int b,
                               int last_valid, void* G, DType out, hipStream_t stream) {
  const dim3 grid((b * b / 4 + kNT - 1) / kNT, (int)nblocks);
  if (out == DType::BF16)
    hipLaunchKernelGGL(split_reduce_kernel<bf16_t>, grid, dim3(kNT), 0, stream, part, nsplit,
                       (int)nblocks, b, last_valid, static_cast<bf16_t*>(G));
  else
    hipLaunchKernelGGL(split_reduce_kernel<float>, grid, dim3(kNT), 0, stream, part, nsplit,
                       (int)nblocks, b, last_valid, static_cast<float*>(G));
  return hipGetLastError();
}

hipError_t launch_pack_skew_grad(const float* M, const void* S, float c, int64_t nblocks, int b,
                                 int last_valid, float sign, float* g_theta, hipStream_t stream) {
  hipLaunchKernelGGL(pack_skew_grad_kernel, dim3((b * b + kNT - 1) / kNT, (int)nblocks), dim3(kNT),
                     0, stream, M, static_cast<const bf16_t*>(S), c, (int)nblocks, b, last_valid,
                     sign, g_theta);
  return hipGetLastError();
}

}  // namespace poetx
