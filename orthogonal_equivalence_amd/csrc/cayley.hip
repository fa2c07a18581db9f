// Exact Cayley map of packed skew generators, and the small kernels of the
// Cayley backward.
//
// Method: skew-symmetric generators Q = -Q^T stored as the strict upper
// triangle (gist.science technical summary of "POET-X: Memory-efficient LLM
// Training by Scaling Orthogonal Transformation", section 2 Methodik,
// Cayley-Neumann parameterisation item). The map used here is the exact
// Cayley map R = (I + Q)(I - Q)^-1 = 2 (I - Q)^-1 - I.
//
// (I - Q)^-1 is formed by blocked Gauss-Jordan elimination without pivoting:
// I - Q has symmetric part I, which is positive definite, so every pivot
// block (a Schur complement of I - Q) again has a positive definite
// symmetric part and is invertible. Three forms, by block size and count:
//   - whole block on one CU (b = 128, and b = 256 from 48 blocks): the tiles
//     in registers, the panels through LDS (cayley_block_kernel);
//   - 2 x 2 pieces of 256 (b = 512 from 48 blocks): the leading piece and
//     its Schur complement inverted by the whole-block kernel, joined by
//     batched float32 products (schur_build);
//   - panels over the chip (every other case), in place in the float32
//     output buffer, each panel of width pw (<= 64) one pair of launches
//     over all blocks at once:
//       prep:   D = A[p][p] inverted in registers (each of 256 threads owns
//               a 4 x 4 piece; four pivots per step, the pivot row and
//               column blocks through LDS, one barrier per step), unless the
//               previous update already did; the workgroup for column tile J
//               writes W_J = Dinv A[p][J] (Dinv itself for J = p, an fp32
//               MFMA product otherwise) to a row-panel buffer and copies
//               A[J][p] to a column-panel buffer;
//       update: every tile (I, J) becomes W_J (I = p) or
//               A[I][J] - colpanel[I] W_J (A[I][p] taken as zero), on MFMA;
//               the tile that becomes the next pivot block is inverted
//               right away (with two or more update workgroups per CU).
//     The last update writes R = 2 B - I and the activation-type copy.
#include "common.h"
#include "kernels.h"

namespace poetx {
namespace {

constexpr int kPW = 64;   // maximum panel width
constexpr int kNT = 256;  // threads per workgroup (a 16 x 16 grid of 4 x 4 pieces)
// 64 x 64 fp32 MFMA operands in LDS: A (A[m][k]) row-major and B (B[k][n])
// stored transposed, both with the k index permuted inside each group of 16
// so that the four k values a lane needs for four consecutive
// v_mfma_f32_16x16x4_f32 steps (k = 16u + 4j + l / 16, j = 0..3) are
// adjacent: one 16-byte LDS read per operand per four MFMAs.
constexpr int kLdP = 68;  // row stride (floats)
__device__ __forceinline__ int kperm(int k) { return (k & ~15) | ((k & 3) << 2) | ((k >> 2) & 3); }
__device__ __forceinline__ int a_off(int m, int k) { return m * kLdP + kperm(k); }
__device__ __forceinline__ int b_off(int k, int n) { return n * kLdP + kperm(k); }

__device__ __forceinline__ int packed_index(int b, int i, int j) {
  // position of (i, j), i < j, in the row-major strict upper triangle
  return i * (2 * b - i - 1) / 2 + (j - i - 1);
}

// A = diag I + sign Q for every block (I - Q for the exact map, Q itself for
// the series); the generators of the last block's rows/columns >= last_valid
// are taken as zero. Piece z (blockIdx.z) is the bo x bo piece of the gb x gb
// matrix starting at row ro[z] and column co[z] (ro == co, or a piece wholly
// on one side of the diagonal; multiples of 32), written to out[z] + blk so
// with row stride ldo; the whole matrix is one piece with gb = bo, ro = co =
// 0. grid (tiles of 32 x 32, nblocks, pieces). A tile below the diagonal
// reads its generators from the mirrored tile above it (coalesced along the
// packed rows) and transposes through LDS.
struct ExpandPieces {
  int ro[3], co[3];
  float diag[3], sign[3];
  float* out[3];
  int64_t ldo, so;
};

constexpr int kExpandTiles = 4;  // 32 x 32 tiles per workgroup, along a tile row

__global__ void __launch_bounds__(kNT)
expand_kernel(const float* __restrict__ theta, int nblocks, int gb, int bo, int last_valid,
              ExpandPieces pc) {
  __shared__ float t[kExpandTiles][32][33];
  const int z = blockIdx.z;
  const int ro = pc.ro[z], co = pc.co[z];
  const float diag = pc.diag[z], sign = pc.sign[z];
  const int ntile = (bo + 31) / 32;
  const int strips = (ntile + kExpandTiles - 1) / kExpandTiles;
  const int TI = blockIdx.x / strips, TJ0 = (blockIdx.x - TI * strips) * kExpandTiles;
  const int blk = blockIdx.y;
  const int r = (blk == nblocks - 1) ? last_valid : gb;
  const float* th = theta + (int64_t)blk * ((int64_t)gb * (gb - 1) / 2);
  float* Ab = pc.out[z] + (int64_t)blk * pc.so;
  const int tx = threadIdx.x & 31, ty0 = threadIdx.x >> 5;  // 8 rows per pass
  // every load of the strip first: for each tile, the upper-triangle tile of
  // its global position (its mirror when it lies below the diagonal), row by row
  float q[kExpandTiles][4];
#pragma unroll
  for (int s = 0; s < kExpandTiles; ++s) {
    const int gi0 = ro + TI * 32, gj0 = co + (TJ0 + s) * 32;
    const bool lower = gi0 > gj0;
    const int ui = lower ? gj0 : gi0, uj = lower ? gi0 : gj0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int i = ui + ty0 + 8 * h, j = uj + tx;
      q[s][h] = (TJ0 + s < ntile && i < j && j < gb && j < r) ? th[packed_index(gb, i, j)] : 0.0f;
    }
  }
#pragma unroll
  for (int s = 0; s < kExpandTiles; ++s)
#pragma unroll
    for (int h = 0; h < 4; ++h) t[s][ty0 + 8 * h][tx] = q[s][h];  // Q[i][j]
  __syncthreads();
#pragma unroll
  for (int s = 0; s < kExpandTiles; ++s) {
    const int TJ = TJ0 + s;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int ty = ty0 + 8 * h;
      const int i = TI * 32 + ty, j = TJ * 32 + tx;
      if (TJ >= ntile || i >= bo || j >= bo) continue;
      const int gi = ro + i, gj = co + j;
      float v;
      if (gi == gj) v = diag;
      else if (gi > gj) v = -sign * t[s][tx][ty];  // Q[i][j] = -Q[j][i]
      else v = sign * t[s][ty][tx];
      Ab[(int64_t)i * pc.ldo + j] = v;
    }
  }
}

// Grid width of expand_kernel for bo x bo pieces.
int expand_grid_x(int bo) {
  const int ntile = (bo + 31) / 32;
  return ntile * ((ntile + kExpandTiles - 1) / kExpandTiles);
}

// The whole b x b matrix as one piece, contiguous blocks.
ExpandPieces whole_piece(int b, float diag, float sign, float* out) {
  ExpandPieces pc{};
  pc.ro[0] = pc.co[0] = 0;
  pc.diag[0] = diag;
  pc.sign[0] = sign;
  pc.out[0] = out;
  pc.ldo = b;
  pc.so = (int64_t)b * b;
  return pc;
}

// Reciprocal: hardware estimate refined by one Newton step (error ~1 ulp).
__device__ __forceinline__ float recip(float x) {
  float r = __builtin_amdgcn_rcpf(x);
  return fmaf(r, fmaf(-x, r, 1.0f), r);
}

// In-place Gauss-Jordan inverse of a 4 x 4 matrix held in registers.
__device__ __forceinline__ void inv4(float m[4][4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float piv = recip(m[k][k]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j != k) m[k][j] *= piv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i == k) continue;
      const float f = m[i][k];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j != k) m[i][j] = fmaf(-f, m[k][j], m[i][j]);
      m[i][k] = -f * piv;
    }
    m[k][k] = piv;
  }
}

// In-place Gauss-Jordan inverse of the leading pw x pw part of a 64 x 64
// matrix distributed as 4 x 4 register pieces (thread (ty, tx) owns rows
// 4ty.., columns 4tx..); entries outside pw x pw must hold the identity.
// Eliminated four pivots at a time: at block step k the pieces of row block
// k and column block k go through LDS (double buffered: one barrier per
// step), every thread inverts the 4 x 4 pivot block D itself and applies
//   a <- base - C' (D^-1 R'),
// with C' = A[i][k] (-I in row block k), R' = A[k][j] (I in column block
// k) and base = a (0 in row or column block k): the row panel becomes
// D^-1 A[k][j], the column panel -A[i][k] D^-1, the pivot block D^-1 and
// every other piece A[i][j] - A[i][k] D^-1 A[k][j].
// buf: 1024 floats of LDS. In a workgroup of more than 256 threads, the
// threads with tid < 256 pass active = true and hold the pieces; every thread
// of the workgroup must call it (it contains workgroup barriers).
__device__ __forceinline__ void gj_invert_regs(float a[4][4], int pw, float* buf,
                                               int tid = (int)threadIdx.x, bool active = true) {
  const int ty = (tid >> 4) & 15, tx = tid & 15;
  for (int k = 0; 4 * k < pw; ++k) {
    float* rb = buf + (k & 1) * 512;  // row-block pieces, by tx
    float* cb = rb + 256;             // column-block pieces, by ty
    if (active && ty == k) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        *reinterpret_cast<float4*>(rb + 16 * tx + 4 * ii) = make_float4(a[ii][0], a[ii][1], a[ii][2], a[ii][3]);
    }
    if (active && tx == k) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        *reinterpret_cast<float4*>(cb + 16 * ty + 4 * ii) = make_float4(a[ii][0], a[ii][1], a[ii][2], a[ii][3]);
    }
    __syncthreads();
    if (!active) continue;
    float d[4][4], r[4][4], c[4][4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const float4 dv = *reinterpret_cast<const float4*>(rb + 16 * k + 4 * ii);
      const float4 rv = *reinterpret_cast<const float4*>(rb + 16 * tx + 4 * ii);
      const float4 cv = *reinterpret_cast<const float4*>(cb + 16 * ty + 4 * ii);
      d[ii][0] = dv.x; d[ii][1] = dv.y; d[ii][2] = dv.z; d[ii][3] = dv.w;
      r[ii][0] = rv.x; r[ii][1] = rv.y; r[ii][2] = rv.z; r[ii][3] = rv.w;
      c[ii][0] = cv.x; c[ii][1] = cv.y; c[ii][2] = cv.z; c[ii][3] = cv.w;
    }
    inv4(d);
    const bool in_row = ty == k, in_col = tx == k;
    // W = D^-1 R'
    float w[4][4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float v = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float rq = in_col ? (q == jj ? 1.0f : 0.0f) : r[q][jj];
          v = fmaf(d[ii][q], rq, v);
        }
        w[ii][jj] = v;
      }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float v = (in_row || in_col) ? 0.0f : a[ii][jj];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float cq = in_row ? (ii == q ? -1.0f : 0.0f) : c[ii][q];
          v = fmaf(-cq, w[q][jj], v);
        }
        a[ii][jj] = v;
      }
  }
  __syncthreads();
}

// acc (this wave's 32 x 32 quadrant of a 64 x 64 product) += A B with both
// operands in the permuted LDS layouts above; fp32 MFMA.
__device__ __forceinline__ void mma64(const float* sA, const float* sB, floatx4 acc[2][2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = (wave >> 1) * 32, c0 = (wave & 1) * 32;
  const int q = 4 * (lane >> 4);
#pragma unroll
  for (int u = 0; u < kPW / 16; ++u) {
    const float4 a0 = *reinterpret_cast<const float4*>(sA + (r0 + (lane & 15)) * kLdP + 16 * u + q);
    const float4 a1 = *reinterpret_cast<const float4*>(sA + (r0 + 16 + (lane & 15)) * kLdP + 16 * u + q);
    const float4 b0 = *reinterpret_cast<const float4*>(sB + (c0 + (lane & 15)) * kLdP + 16 * u + q);
    const float4 b1 = *reinterpret_cast<const float4*>(sB + (c0 + 16 + (lane & 15)) * kLdP + 16 * u + q);
    const float av0[4] = {a0.x, a0.y, a0.z, a0.w}, av1[4] = {a1.x, a1.y, a1.z, a1.w};
    const float bv0[4] = {b0.x, b0.y, b0.z, b0.w}, bv1[4] = {b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(av0[j], bv0[j], acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av0[j], bv1[j], acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(av1[j], bv0[j], acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av1[j], bv1[j], acc[1][1], 0, 0, 0);
    }
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

// grid (b / pw column tiles, nblocks). dinv (optional): the pivot block's
// inverse (64 x 64 per block, identity outside pw x pw), inverted by the
// previous panel's update; without it every workgroup inverts the pivot.
__global__ void __launch_bounds__(kNT)
panel_prep_kernel(const float* __restrict__ A, int b, int pw, int p,
                  float* __restrict__ rowbuf, float* __restrict__ colbuf,
                  const float* __restrict__ dinv) {
  __shared__ __attribute__((aligned(16))) float sD[kPW * kLdP];
  __shared__ __attribute__((aligned(16))) float sX[kPW * kLdP];
  __shared__ __attribute__((aligned(16))) float gjbuf[1024];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int J = blockIdx.x;
  const int64_t blk = blockIdx.y;
  const float* Ab = A + blk * (int64_t)b * b;
  const int p0 = p * pw, j0 = J * pw;

  // all loads first, from clamped (always valid) addresses, then the selects
  // and stores: no load waits behind a store or a branch
  float av[4][4], cv[4][4], xv[4][4];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int gi = min(4 * ty + ii, pw - 1), gj = min(4 * tx + jj, pw - 1);
      av[ii][jj] = dinv ? dinv[blk * kPW * kPW + (4 * ty + ii) * kPW + 4 * tx + jj]
                        : Ab[(int64_t)(p0 + gi) * b + p0 + gj];
      cv[ii][jj] = Ab[(int64_t)(j0 + gi) * b + p0 + gj];
      xv[ii][jj] = Ab[(int64_t)(p0 + gi) * b + j0 + gj];
    }
  float a[4][4];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int gi = 4 * ty + ii, gj = 4 * tx + jj;
      const bool in = gi < pw && gj < pw;
      a[ii][jj] = (in || dinv) ? av[ii][jj] : (gi == gj ? 1.0f : 0.0f);
      if (in) colbuf[(blk * b + j0 + gi) * pw + gj] = cv[ii][jj];
      if (J != p) sX[b_off(gi, gj)] = in ? xv[ii][jj] : 0.0f;
    }
  if (!dinv) gj_invert_regs(a, pw, gjbuf);

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
    for (int jj = 0; jj < 4; ++jj) sD[a_off(4 * ty + ii, 4 * tx + jj)] = a[ii][jj];
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
// dinv_next (optional, not with `final`): the workgroup that updates the next
// pivot block (p + 1, p + 1) also inverts it and writes the inverse there
// (64 x 64 per block, identity outside pw x pw), for the next prep launch.
// Those workgroups take the first ids (one per block), so the inversions run
// beside the other tiles' updates.
__global__ void __launch_bounds__(kNT)
panel_update_kernel(float* __restrict__ A, int b, int pw, int p,
                    const float* __restrict__ rowbuf, const float* __restrict__ colbuf,
                    int final, bf16_t* __restrict__ act_out, float* __restrict__ dinv_next) {
  __shared__ __attribute__((aligned(16))) float sC[kPW * kLdP];
  __shared__ __attribute__((aligned(16))) float sW[kPW * kLdP];
  __shared__ __attribute__((aligned(16))) float gjbuf[1024];
  const int tid = threadIdx.x;
  const int nt = b / pw;
  int tile = blockIdx.x;
  int64_t blk = blockIdx.y;
  if (dinv_next) {
    const int per = nt * nt, nb = (int)gridDim.y;
    const int64_t lin = (int64_t)blockIdx.y * per + blockIdx.x;
    const int piv = (p + 1) * nt + (p + 1);
    if (lin < nb) {
      blk = lin;
      tile = piv;
    } else {
      const int64_t rest = lin - nb;
      blk = rest / (per - 1);
      const int t = (int)(rest - blk * (per - 1));
      tile = t < piv ? t : t + 1;
    }
  }
  const int I = tile / nt, J = tile - (tile / nt) * nt;
  const bool next_pivot = dinv_next && I == p + 1 && J == p + 1;
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
    float v[kPW * kPW / kNT];  // all loads before the stores
#pragma unroll
    for (int t = 0; t < kPW * kPW / kNT; ++t) {
      const int e = tid + t * kNT, gi = min(e >> 6, pw - 1), gj = min(e & 63, pw - 1);
      v[t] = rb[(int64_t)gi * b + j0 + gj];
    }
#pragma unroll
    for (int t = 0; t < kPW * kPW / kNT; ++t) {
      const int e = tid + t * kNT, gi = e >> 6, gj = e & 63;
      if (gi < pw && gj < pw) emit(gi, gj, v[t]);
    }
    return;
  }
  {
    // each thread stages a 4 x 4 piece of C (column panel rows I) and W (row
    // panel columns J): all loads first, from clamped (always valid)
    // addresses, then the LDS stores
    const int ty = tid >> 4, tx = tid & 15;
    float cv[4][4], wv[4][4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int gi = min(4 * ty + ii, pw - 1), gj = min(4 * tx + jj, pw - 1);
        cv[ii][jj] = cb[(int64_t)(i0 + gi) * pw + gj];
        wv[ii][jj] = rb[(int64_t)gi * b + j0 + gj];
      }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int gi = 4 * ty + ii, gj = 4 * tx + jj;
        const bool in = gi < pw && gj < pw;
        sC[a_off(gi, gj)] = in ? cv[ii][jj] : 0.0f;
        sW[b_off(gi, gj)] = in ? wv[ii][jj] : 0.0f;
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
  if (!next_pivot) return;  // uniform across the workgroup
  // the new pivot block, row-major through LDS into 4 x 4 register pieces
  __syncthreads();  // every wave is done reading sC
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sC[mma_row(mi, e) * kLdP + mma_col(ni)] = base[mi][ni][e] - acc[mi][ni][e];
  __syncthreads();
  const int ty = tid >> 4, tx = tid & 15;
  float a[4][4];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int gi = 4 * ty + ii, gj = 4 * tx + jj;
      a[ii][jj] = (gi < pw && gj < pw) ? sC[gi * kLdP + gj] : (gi == gj ? 1.0f : 0.0f);
    }
  gj_invert_regs(a, pw, gjbuf);
  float* dn = dinv_next + blk * kPW * kPW;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
    *reinterpret_cast<float4*>(dn + (4 * ty + ii) * kPW + 4 * tx) =
        make_float4(a[ii][0], a[ii][1], a[ii][2], a[ii][3]);
}

// ---- whole block per workgroup: b = 64 NT, NT = 2 or 4 ----
// The block stays on one CU from the generators to R. Each wave owns TPW of
// the NT x NT 64 x 64 tiles in registers, in the layout of the fp32 MFMA
// accumulators (tile element (16 mi + 4 (lane / 16) + e, 16 ni + lane % 16)
// is acc[mi][ni][e]); the blocked Gauss-Jordan elimination runs panel by
// panel with the pivot block inverted by the first 256 threads in 4 x 4
// register pieces (gj_invert_regs) and every 64 x 64 x 64 product on MFMA:
//   pivot      D = A[p][p]          -> D^-1
//   column     A[I][p] (= C_I)      -> C'_I = -C_I D^-1
//   row        A[p][J]              -> D^-1 A[p][J]
//   the rest   A[I][J]              -> A[I][J] + C'_I A[p][J]
// The column panel goes first; the row panel and the rest then all read the
// row panel as published, so they run together (three 64 x 64 x 64 products
// per SIMD for NT = 4, against two then three when the rest waits for the
// new row panel). LDS holds D^-1 in both operand layouts, the row panel
// (B layout) and the column panel (A layout: -C_I, then C'_I).

// acc[mi][ni] += A B for one wave's full 64 x 64 tile, K = 64, operands in
// the permuted LDS layouts of a_off / b_off.
__device__ __forceinline__ void wave_mma64(const float* sA, const float* sB, floatx4 acc[4][4],
                                           int lane) {
  const int q = 4 * (lane >> 4);
#pragma unroll
  for (int u = 0; u < kPW / 16; ++u) {
    float4 av[4], bv[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
      av[mi] = *reinterpret_cast<const float4*>(sA + (16 * mi + (lane & 15)) * kLdP + 16 * u + q);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
      bv[ni] = *reinterpret_cast<const float4*>(sB + (16 * ni + (lane & 15)) * kLdP + 16 * u + q);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const float a = j == 0 ? av[mi].x : j == 1 ? av[mi].y : j == 2 ? av[mi].z : av[mi].w;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const float bb = j == 0 ? bv[ni].x : j == 1 ? bv[ni].y : j == 2 ? bv[ni].z : bv[ni].w;
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, acc[mi][ni], 0, 0, 0);
        }
      }
    }
  }
}

__device__ __forceinline__ int tile_row(int mi, int e, int lane) { return 16 * mi + 4 * (lane >> 4) + e; }
__device__ __forceinline__ int tile_col(int ni, int lane) { return 16 * ni + (lane & 15); }

template <int NT> struct BlockShape {
  static constexpr int B = 64 * NT;
  static constexpr int WAVES = NT * NT / 2 > 4 ? NT * NT / 2 : 4;
  static constexpr int TPW = NT * NT / WAVES;  // tiles per wave
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int TILE = kPW * kLdP;      // floats of one 64 x 64 operand tile
  // D^-1 twice, the row and column panels, the pivot-inversion buffer
  static constexpr int LDS = (2 + 2 * (NT - 1)) * TILE + 1024;
  static_assert(WAVES * TILE <= LDS, "per-wave staging tiles must fit");
};

// Tile (I, J) held in slot s of a wave. Waves go to the four SIMDs round
// robin; for NT = 4 the SIMD of tile (I, J) is (I + J) mod 4, so every SIMD
// owns one tile of each tile row and column and a panel's trailing update
// (the tiles outside row and column p) puts at most three tiles on a SIMD.
template <int NT>
__device__ __forceinline__ void tile_of(int wave, int s, int& I, int& J) {
  if constexpr (NT == 4) {
    I = 2 * (wave >> 2) + s;
    J = ((wave & 3) - I) & 3;
  } else {
    const int q = wave * BlockShape<NT>::TPW + s;
    I = q / NT;
    J = q % NT;
  }
}

// grid (nblocks); R = 2 A^-1 - I (float32) to out + blk so (row stride ldo)
// and, when act is given, its bf16 copy at the same offsets in act. A is
// I - Q for the leading B x B piece of the gb x gb generator blocks in theta
// (gb = B: the whole block), or, when dense is not null, the float32 matrix
// at dense + blk si (B x B, row stride ldi).
template <int NT>
__global__ void __launch_bounds__(BlockShape<NT>::THREADS)
cayley_block_kernel(const float* __restrict__ theta, const float* __restrict__ dense, int64_t ldi,
                    int64_t si, int nblocks, int last_valid, int gb, float* __restrict__ out,
                    int64_t ldo, int64_t so, bf16_t* __restrict__ act) {
  typedef BlockShape<NT> S;
  constexpr int B = S::B, TPW = S::TPW, TILE = S::TILE;
  __shared__ __attribute__((aligned(16))) float lds[S::LDS];
  float* const sDa = lds;                    // D^-1, A-operand layout (and D, row-major)
  float* const sDb = lds + TILE;             // D^-1, B-operand layout
  float* const sW = lds + 2 * TILE;          // row panel, B layout, NT - 1 tiles
  float* const sC = sW + (NT - 1) * TILE;    // negated column panel, A layout
  float* const gjbuf = sC + (NT - 1) * TILE;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* const stage = lds + wave * TILE;    // this wave's 64 x 68 staging tile (start, end)
  const int blk = blockIdx.x;
  const int r = (blk == nblocks - 1) ? last_valid : gb;
  const bool dense_in = dense != nullptr;
  const float* th = dense_in ? nullptr : theta + (int64_t)blk * ((int64_t)gb * (gb - 1) / 2);

  floatx4 t[TPW][4][4];
  if (dense_in) {
    // A row by row (lane l reads column l) through the wave's staging tile
    // into the accumulator layout
    const float* src = dense + (int64_t)blk * si;
#pragma unroll
    for (int s = 0; s < TPW; ++s) {
      int I, J;
      tile_of<NT>(wave, s, I, J);
      const float* ts = src + (64 * I) * ldi + 64 * J + lane;
#pragma unroll 1
      for (int c = 0; c < 64; c += 16) {  // 16 rows in flight at a time
        float g[16];
#pragma unroll
        for (int row = 0; row < 16; ++row) g[row] = ts[(c + row) * ldi];
#pragma unroll
        for (int row = 0; row < 16; ++row) stage[(c + row) * kLdP + lane] = g[row];
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            t[s][mi][ni][e] = stage[tile_row(mi, e, lane) * kLdP + tile_col(ni, lane)];
    }
  } else {
    // A = I - Q from the packed generators (those of rows / columns >= r
    // read as 0). Every tile stages the upper-triangle tile of its position,
    // (min(I, J), max(I, J)), one row per load instruction: lane l reads
    // column l, so a row is 64 consecutive generators (its packed index is
    // rowbase(i) + j with rowbase uniform across the wave). The tile then
    // takes -theta(i, j) above the diagonal and +theta(j, i) (the staged
    // transpose) below it: (I - Q)[i][j] = theta(j, i) for i > j.
#pragma unroll
    for (int s = 0; s < TPW; ++s) {
      int I, J;
      tile_of<NT>(wave, s, I, J);
      const int R0 = 64 * (I < J ? I : J), C0 = 64 * (I < J ? J : I);
      const int j = C0 + lane;
      float g[64];  // all 64 row loads in flight before the first LDS store
#pragma unroll
      for (int row = 0; row < 64; ++row) {
        const int i = R0 + row;
        const int rowbase = i * (2 * gb - i - 1) / 2 - i - 1;
        g[row] = (i < j && j < r) ? th[rowbase + j] : 0.0f;
      }
#pragma unroll
      for (int row = 0; row < 64; ++row) stage[row * kLdP + lane] = g[row];
      const bool diag = I == J, lower = I > J;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int rr = tile_row(mi, e, lane), cc = tile_col(ni, lane);
            float v;
            if (diag) v = rr == cc ? 1.0f : rr < cc ? -stage[rr * kLdP + cc] : stage[cc * kLdP + rr];
            else if (lower) v = stage[cc * kLdP + rr];
            else v = -stage[rr * kLdP + cc];
            t[s][mi][ni][e] = v;
          }
    }
  }
  __syncthreads();  // the staging tiles overlap the panel buffers

  for (int p = 0; p < NT; ++p) {
    // publish the pivot block (row-major), the row panel (B layout) and the
    // negated column panel (A layout)
#pragma unroll
    for (int s = 0; s < TPW; ++s) {
      int I, J;
      tile_of<NT>(wave, s, I, J);
      if (I != p && J != p) continue;
      float* dst = (I == p && J == p) ? sDa
                 : (I == p) ? sW + (J < p ? J : J - 1) * TILE
                            : sC + (I < p ? I : I - 1) * TILE;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int rr = tile_row(mi, e, lane), cc = tile_col(ni, lane);
            const float v = t[s][mi][ni][e];
            if (I == p && J == p) dst[rr * kLdP + cc] = v;
            else if (I == p) dst[b_off(rr, cc)] = v;
            else dst[a_off(rr, cc)] = -v;
          }
    }
    __syncthreads();

    // D^-1 by the first 256 threads, written in both operand layouts
    {
      const bool active = tid < 256;
      const int ty = (tid >> 4) & 15, tx = tid & 15;
      float a[4][4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) a[ii][jj] = active ? sDa[(4 * ty + ii) * kLdP + 4 * tx + jj] : 0.0f;
      gj_invert_regs(a, kPW, gjbuf, tid, active);
      if (active) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            sDa[a_off(4 * ty + ii, 4 * tx + jj)] = a[ii][jj];
            sDb[b_off(4 * ty + ii, 4 * tx + jj)] = a[ii][jj];
          }
      }
    }
    __syncthreads();

    // column panel C'_I = -A[I][p] D^-1 (sC holds -A[I][p]) and the pivot
    // block D^-1; the wave of tile (I, p) is the only reader of sC tile I, so
    // it overwrites it with C'_I once its product is done
#pragma unroll
    for (int s = 0; s < TPW; ++s) {
      int I, J;
      tile_of<NT>(wave, s, I, J);
      if (J != p) continue;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) t[s][mi][ni] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (I == p) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              t[s][mi][ni][e] = sDa[a_off(tile_row(mi, e, lane), tile_col(ni, lane))];
      } else {
        float* cp = sC + (I < p ? I : I - 1) * TILE;
        wave_mma64(cp, sDb, t[s], lane);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              cp[a_off(tile_row(mi, e, lane), tile_col(ni, lane))] = t[s][mi][ni][e];
      }
    }
    __syncthreads();

    // row panel W_J = D^-1 A[p][J] and trailing update A[I][J] += C'_I A[p][J],
    // both from the row panel as published
#pragma unroll
    for (int s = 0; s < TPW; ++s) {
      int I, J;
      tile_of<NT>(wave, s, I, J);
      if (J == p) continue;
      if (I == p) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) t[s][mi][ni] = floatx4{0.f, 0.f, 0.f, 0.f};
        wave_mma64(sDa, sW + (J < p ? J : J - 1) * TILE, t[s], lane);
      } else {
        wave_mma64(sC + (I < p ? I : I - 1) * TILE, sW + (J < p ? J : J - 1) * TILE, t[s], lane);
      }
    }
    __syncthreads();  // panels are rewritten by the next step (and by the staging below)
  }

  // R = 2 (I - Q)^-1 - I, staged row-major so that rows leave as 16-byte
  // (float32) and 8-byte (bf16) vectors
  float* ob = out + (int64_t)blk * so;
  bf16_t* ab = act ? act + (int64_t)blk * so : nullptr;
#pragma unroll
  for (int s = 0; s < TPW; ++s) {
    int I, J;
    tile_of<NT>(wave, s, I, J);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = tile_row(mi, e, lane), cc = tile_col(ni, lane);
          stage[rr * kLdP + cc] = 2.0f * t[s][mi][ni][e] - (64 * I + rr == 64 * J + cc ? 1.0f : 0.0f);
        }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int rr = 4 * q + (lane >> 4), c4 = 4 * (lane & 15);
      const float4 v = *reinterpret_cast<const float4*>(stage + rr * kLdP + c4);
      const int64_t off = (int64_t)(64 * I + rr) * ldo + 64 * J + c4;
      *reinterpret_cast<float4*>(ob + off) = v;
      if (ab) {
        union { uint2 u; bf16_t h[4]; } o;
        o.h[0] = f32_to_bf16(v.x); o.h[1] = f32_to_bf16(v.y);
        o.h[2] = f32_to_bf16(v.z); o.h[3] = f32_to_bf16(v.w);
        *reinterpret_cast<uint2*>(ab + off) = o.u;
      }
    }
  }
}

// grid (ceil(b*b / (4 kNT)), nblocks); b*b is a multiple of 4. col_scale
// (optional) multiplies column j of block blk by col_scale[blk b + j].
// sub > 1: the partials are grams of (sub b) x (sub b) super blocks (sub
// consecutive blocks each) and block blk is the diagonal piece
// (blk % sub) of super block blk / sub.
template <typename TOut>
__global__ void __launch_bounds__(kNT)
split_reduce_kernel(const float* __restrict__ part, int nsplit, int nblocks, int b,
                    int last_valid, const float* __restrict__ col_scale, TOut* __restrict__ G,
                    int sub) {
  const int q = blockIdx.x * kNT + threadIdx.x;  // float4 index within the block
  const int bb = b * b;
  if (4 * q >= bb) return;
  const int blk = blockIdx.y;
  const int64_t total = (int64_t)nblocks * bb * sub;  // floats of one split's partials
  const int64_t off = (int64_t)blk * bb + 4 * q;
  const int ld = b * sub, piece = (blk % sub) * b;
  const int i0 = (4 * q) / b, j0 = (4 * q) % b;
  const int64_t src = ((int64_t)(blk / sub) * ld + piece + i0) * ld + piece + j0;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < nsplit; ++s) {
    const float4 t = *reinterpret_cast<const float4*>(part + (int64_t)s * total + src);
    v.x += t.x; v.y += t.y; v.z += t.z; v.w += t.w;
  }
  float e[4] = {v.x, v.y, v.z, v.w};
  if (col_scale) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int j = (4 * q + t) % b;
      const int valid = (blk == nblocks - 1) ? last_valid : b;
      e[t] *= (j < valid) ? col_scale[(int64_t)blk * b + j] : 0.0f;
    }
  }
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

// g_theta(i, j) = sign ((M + c S)[i][j] - (M + c S)[j][i]), S optional (bf16).
// grid (nt (nt + 1) / 2 tile pairs, nblocks), nt = ceil(b / 32): the workgroup
// for the upper tile (TI, TJ), TI <= TJ, reads it and its mirror (TJ, TI)
// row by row (coalesced) into LDS and writes the packed entries of (TI, TJ),
// which are contiguous along j for each row i.
// grid.y covers the blocks of the first set, then those of the second.
__global__ void __launch_bounds__(kNT)
pack_skew_grad_kernel(PackSet s1, PackSet s2, float c, int b, float sign) {
  __shared__ float up[32][33], lo[32][33];
  const int nt = (b + 31) / 32;
  int p = blockIdx.x, TI = 0;
  while (p >= nt - TI) {  // tile pair p -> (TI, TJ), row by row of the upper triangle
    p -= nt - TI;
    ++TI;
  }
  const int TJ = TI + p;
  const bool second = blockIdx.y >= s1.nblocks;
  const float* __restrict__ M = second ? s2.M : s1.M;
  const bf16_t* __restrict__ S = static_cast<const bf16_t*>(second ? s2.S : s1.S);
  float* __restrict__ g = second ? s2.g_theta : s1.g_theta;
  const int nblocks = (int)(second ? s2.nblocks : s1.nblocks);
  const int blk = second ? (int)(blockIdx.y - s1.nblocks) : (int)blockIdx.y;
  const int r = (blk == nblocks - 1) ? (second ? s2.last_valid : s1.last_valid) : b;
  const int64_t base = (int64_t)blk * b * b;
  const int tx = threadIdx.x & 31, ty0 = threadIdx.x >> 5;
  for (int ty = ty0; ty < 32; ty += 8) {
    const int i = TI * 32 + ty, j = TJ * 32 + tx;      // (TI, TJ)
    const int i2 = TJ * 32 + ty, j2 = TI * 32 + tx;    // (TJ, TI)
    float u = 0.0f, l = 0.0f;
    if (i < b && j < b) {
      const int64_t a = base + (int64_t)i * b + j;
      u = M[a];
      if (S) u += c * bf16_to_f32(S[a]);
    }
    if (i2 < b && j2 < b) {
      const int64_t a = base + (int64_t)i2 * b + j2;
      l = M[a];
      if (S) l += c * bf16_to_f32(S[a]);
    }
    up[ty][tx] = u;
    lo[ty][tx] = l;
  }
  __syncthreads();
  float* gb = g + (int64_t)blk * (b * (b - 1) / 2);
  for (int ty = ty0; ty < 32; ty += 8) {
    const int i = TI * 32 + ty, j = TJ * 32 + tx;
    if (i >= j || j >= b) continue;
    // (M + c S)[j][i] = lo[j - 32 TJ][i - 32 TI]
    gb[packed_index(b, i, j)] = (j < r) ? sign * (up[ty][tx] - lo[tx][ty]) : 0.0f;
  }
}

// Blocks of 512 as 2 x 2 pieces of 256 (Schur complement), for many blocks.
// With A = I - Q = [[A11, A12], [A21, A22]] (A11 = I - Q11, A12 = -Q12,
// A21 = Q12^T, A22 = I - Q22), Z = A11^-1, X = Z Q12 and V = -A21 Z = Q21 Z:
//   S = A22 - A21 Z A12 = (I - Q22) - V Q12,
//   A^-1 = [[Z + X S^-1 V, X S^-1], [S^-1 V, S^-1]].
// The two inversions run on the whole-block kernel, which returns T = 2 Z - I
// and R22 = 2 S^-1 - I directly; with Z = (T + I) / 2 and S^-1 = (R22 + I) / 2
// the pieces of R = 2 A^-1 - I are
//   R12 = X R22 + X,   R21 = R22 V + V,   R11 = T + R12 V,
// each a 256 x 256 float32 product of all blocks in a batched launch; X and V,
// and then R12 and R21, are independent products with the same scale factors,
// so each pair shares one launch. A11
// and S have positive definite symmetric parts (I, and a Schur complement of
// a matrix whose symmetric part is I), so neither elimination pivots.
constexpr int kSchurMinBlocks = 48;

// (The same form for 72 blocks of 256, on pieces of 128, took 211 us against
// 187 us for the whole-block kernel, so b = 256 keeps that kernel.)
bool use_schur(int64_t nblocks, int b) { return b == 512 && nblocks >= kSchurMinBlocks; }

// NT: the whole-block kernel's tile count per edge for the pieces (H = 64 NT,
// B = 2 H).
template <int NT>
hipError_t schur_build(const float* theta, int nb, int last_valid, float* R, bf16_t* act,
                       float* ws, hipStream_t stream) {
  constexpr int H = 64 * NT, B = 2 * H;
  constexpr int64_t BB = (int64_t)B * B;
  // Every piece lives in a B x B frame per block (row stride B, block
  // stride B^2), as the pieces of R do, so that the paired products share
  // their strides: W1 holds T, Q12, Q21 and I - Q22 in its four quadrants,
  // W2 holds V and S in its top half, and X sits in R's R11 quadrant until
  // R11 is written.
  float* W1 = ws;
  float* W2 = ws + nb * BB;
  float* T = W1;
  float* Q12 = W1 + H;
  float* Q21 = W1 + H * B;
  float* D22 = W1 + H * B + H;
  float* V = W2;
  float* S = W2 + H;
  float* X = R;
  float* R12 = R + H;
  float* R21 = R + H * B;
  float* R22 = R + H * B + H;
  hipError_t e;
  ExpandPieces pc{};
  pc.ro[0] = 0; pc.co[0] = H; pc.diag[0] = 0.0f; pc.sign[0] = 1.0f; pc.out[0] = Q12;   // Q12
  pc.ro[1] = H; pc.co[1] = 0; pc.diag[1] = 0.0f; pc.sign[1] = 1.0f; pc.out[1] = Q21;   // Q21
  pc.ro[2] = H; pc.co[2] = H; pc.diag[2] = 1.0f; pc.sign[2] = -1.0f; pc.out[2] = D22;  // I - Q22
  pc.ldo = B;
  pc.so = BB;
  hipLaunchKernelGGL(expand_kernel, dim3(expand_grid_x(H), nb, 3), dim3(kNT), 0, stream, theta, nb,
                     B, H, last_valid, pc);
  hipLaunchKernelGGL(cayley_block_kernel<NT>, dim3((unsigned)nb), dim3(BlockShape<NT>::THREADS),
                     0, stream, theta, nullptr, (int64_t)0, (int64_t)0, nb, last_valid, B, T,
                     (int64_t)B, BB, nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // C = alpha A B + beta D per block (A row-major, B(n, k) = Bm[k][n]), every
  // operand with row stride 512 and block stride 512^2; a second job of the
  // same shape runs in the same launch
  auto prod = [&](const float* A, const float* Bm, float alpha, const float* D, float beta,
                  float* C, const float* A2, const float* B2, const float* D2, float* C2,
                  bf16_t* C_act = nullptr, bf16_t* C2_act = nullptr) {
    GemmParams g;
    g.A = A; g.B = Bm; g.C = C; g.D = D;
    g.lda = g.ldb = g.ldc = g.ldd = B;
    g.sA = g.sB = g.sC = g.sD = BB;
    g.M = g.N = g.K = g.M_last = g.N_last = g.K_last = H;
    g.batch = A2 ? 2 * nb : nb;
    g.kchunk = H;
    g.alpha = alpha; g.beta = beta;
    g.C_act = C_act;
    if (A2) {
      g.batch_split = nb;
      g.A2 = A2; g.B2 = B2; g.C2 = C2; g.D2 = D2;
      g.C2_act = C2_act;
    }
    return launch_gemm(DType::F32, DType::F32, true, false, g, stream);
  };
  // X = Z Q12 = (T Q12 + Q12) / 2 and V = Q21 Z = (Q21 T + Q21) / 2
  if ((e = prod(T, Q12, 0.5f, Q12, 0.5f, X, Q21, T, Q21, V)) != hipSuccess) return e;
  // S = (I - Q22) - V Q12
  if ((e = prod(V, Q12, -1.0f, D22, 1.0f, S, nullptr, nullptr, nullptr, nullptr)) != hipSuccess)
    return e;
  // R22 = 2 S^-1 - I, written into the block with its bf16 copy
  hipLaunchKernelGGL(cayley_block_kernel<NT>, dim3((unsigned)nb), dim3(BlockShape<NT>::THREADS),
                     0, stream, nullptr, S, (int64_t)B, BB, nb, last_valid, B, R22, (int64_t)B, BB,
                     act ? act + H * B + H : nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // R12 = X R22 + X and R21 = R22 V + V in one launch, then R11 = T + R12 V
  // (over X, which nothing reads any more); each with its bf16 copy
  if ((e = prod(X, R22, 1.0f, X, 1.0f, R12, R22, V, V, R21, act ? act + H : nullptr,
                act ? act + H * B : nullptr)) != hipSuccess)
    return e;
  return prod(R12, V, 1.0f, T, 1.0f, R, nullptr, nullptr, nullptr, nullptr, act);
}

}  // namespace

int cayley_panel_width(int b) {
  if (b <= kPW) return b;
  int pw = kPW;
  while (b % pw) pw >>= 1;
  return pw;
}

size_t cayley_workspace_floats(int64_t nblocks, int b) {
  if (use_schur(nblocks, b)) return 2 * (size_t)nblocks * b * b;
  const int pw = cayley_panel_width(b);
  // row and column panels, and the next pivot block's inverse
  return 2 * (size_t)nblocks * (size_t)pw * (size_t)b + (size_t)nblocks * kPW * kPW;
}

hipError_t launch_cayley_build(const float* theta, int64_t nblocks, int b, int last_valid,
                               float* blocks_f32, void* blocks_act, DType act, float* ws,
                               hipStream_t stream) {
  bf16_t* act_bf16 = (act == DType::BF16) ? static_cast<bf16_t*>(blocks_act) : nullptr;
  // The whole-block kernel takes about the same time for any number of blocks
  // up to one per CU (its latency is the elimination's sequence of pivots on
  // one CU); the panel kernels spread every block's products over the chip, so
  // with few blocks of 256 they finish first (measured: 16 blocks 164 -> 119
  // us, 32 blocks 172 -> 140 us), with 64 or more the whole-block kernel does.
  if (use_schur(nblocks, b))
    return schur_build<4>(theta, (int)nblocks, last_valid, blocks_f32, act_bf16, ws, stream);
  const bool whole_block = b == 128 || (b == 256 && nblocks >= 48);
  if (whole_block) {  // the whole block on one CU
    if (b == 256)
      hipLaunchKernelGGL(cayley_block_kernel<4>, dim3((unsigned)nblocks),
                         dim3(BlockShape<4>::THREADS), 0, stream, theta, nullptr, (int64_t)0,
                         (int64_t)0, (int)nblocks, last_valid, b, blocks_f32, (int64_t)b,
                         (int64_t)b * b, act_bf16);
    else
      hipLaunchKernelGGL(cayley_block_kernel<2>, dim3((unsigned)nblocks),
                         dim3(BlockShape<2>::THREADS), 0, stream, theta, nullptr, (int64_t)0,
                         (int64_t)0, (int)nblocks, last_valid, b, blocks_f32, (int64_t)b,
                         (int64_t)b * b, act_bf16);
    return hipGetLastError();
  }
  const int pw = cayley_panel_width(b);
  const int nt = b / pw;
  const int nb = (int)nblocks;
  float* rowbuf = ws;
  float* colbuf = ws + (size_t)nblocks * pw * b;
  float* dinv = colbuf + (size_t)nblocks * pw * b;
  bf16_t* act_out = (act == DType::BF16) ? static_cast<bf16_t*>(blocks_act) : nullptr;
  hipLaunchKernelGGL(expand_kernel, dim3(expand_grid_x(b), nb, 1), dim3(kNT), 0, stream, theta, nb,
                     b, b, last_valid, whole_piece(b, 1.0f, -1.0f, blocks_f32));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // With at least two update workgroups per CU, the next pivot's inversion
  // runs in the update launch beside the other tiles (8 blocks of 1024:
  // build 827 -> 662 us; 16 of 512: 327 -> 304 us); with one round of
  // workgroups it would only lengthen the launch, so prep inverts it.
  const bool early_pivot = (int64_t)nt * nt * nb >= 512;
  for (int p = 0; p < nt; ++p) {
    const bool take = early_pivot && p > 0, give = early_pivot && p < nt - 1;
    hipLaunchKernelGGL(panel_prep_kernel, dim3(nt, nb), dim3(kNT), 0, stream, blocks_f32, b, pw, p,
                       rowbuf, colbuf, take ? (const float*)dinv : nullptr);
    hipLaunchKernelGGL(panel_update_kernel, dim3(nt * nt, nb), dim3(kNT), 0, stream, blocks_f32, b,
                       pw, p, rowbuf, colbuf, (int)(p == nt - 1), act_out, give ? dinv : nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_expand_skew(const float* theta, int64_t nblocks, int b, int last_valid,
                              float diag, float sign, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(expand_kernel, dim3(expand_grid_x(b), (int)nblocks, 1), dim3(kNT), 0, stream,
                     theta, (int)nblocks, b, b, last_valid, whole_piece(b, diag, sign, out));
  return hipGetLastError();
}

hipError_t launch_split_reduce(const float* part, int nsplit, int64_t nblocks, int b,
                               int last_valid, void* G, DType out, hipStream_t stream,
                               const float* col_scale, int sub) {
  if (sub < 1 || nblocks % sub != 0 || (sub > 1 && last_valid != b)) return hipErrorInvalidValue;
  const dim3 grid((b * b / 4 + kNT - 1) / kNT, (int)nblocks);
  if (out == DType::BF16)
    hipLaunchKernelGGL(split_reduce_kernel<bf16_t>, grid, dim3(kNT), 0, stream, part, nsplit,
                       (int)nblocks, b, last_valid, col_scale, static_cast<bf16_t*>(G), sub);
  else
    hipLaunchKernelGGL(split_reduce_kernel<float>, grid, dim3(kNT), 0, stream, part, nsplit,
                       (int)nblocks, b, last_valid, col_scale, static_cast<float*>(G), sub);
  return hipGetLastError();
}

hipError_t launch_pack_skew_grad(const PackSet& a, const PackSet* b2, float c, int b, float sign,
                                 hipStream_t stream) {
  const int nt = (b + 31) / 32;
  const PackSet none{nullptr, nullptr, 0, 0, nullptr};
  const int64_t total = a.nblocks + (b2 ? b2->nblocks : 0);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_skew_grad_kernel, dim3(nt * (nt + 1) / 2, (unsigned)total), dim3(kNT), 0,
                     stream, a, b2 ? *b2 : none, c, b, sign);
  return hipGetLastError();
}

}  // namespace poetx
