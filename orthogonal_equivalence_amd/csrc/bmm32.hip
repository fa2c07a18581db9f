// Batched square float32 products C = alpha A B + beta D on fp32 MFMA (and,
// when asked, C's bf16 copy), for the
// b x b block products of the Cayley build (the 2 x 2 Schur pieces) and of
// the Cayley-Neumann series and its VJP (b a multiple of 128).
//
// One workgroup of four waves (one per SIMD) per 128 x TN output tile (TN =
// 128, or 64 when 128-wide tiles would leave the last round of workgroups
// mostly empty), each wave a 64 x TN/2 quarter of v_mfma_f32_16x16x4_f32
// tiles. The K
// extent streams through a 4-slot LDS ring in 32-deep K tiles copied with
// global_load_lds_dwordx4, three tiles ahead of the products, so the loads'
// latency is hidden behind 64 products per wave per tile (the register-staged
// generic GEMM left its waves waiting on memory more than half the time at
// these sizes). The swizzles below are chosen so that the fragment reads of a
// 16-lane group hit distinct banks of gfx950's 64-bank LDS.
//
// Fragments: the 16x16x4 product takes from lane l the A entry (row l % 16,
// k = l / 16) and the B entry (k = l / 16, column l % 16). Inside each group
// of 16 k, product j of four gives lane group q = l / 16 the k index
// 4 q + j, so a lane's four A values are one 16-byte LDS read (four
// consecutive k of its row); the k order inside the sum changes, not its terms.
#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace poetx {
namespace {

constexpr int kT = 256;                  // threads
constexpr int kTile = 128;               // output tile rows (and the shape granule)
constexpr int kBK = 32;                  // K tile depth (floats)
constexpr int kRing = 4;

// A tile: 128 rows of 8 16-byte chunks; LDS chunk (r, cl) holds the row's
// global chunk cl ^ swz_a(r). B tile: 32 rows (k) of TN / 4 chunks (n); LDS
// chunk (k, cl) holds global chunk cl ^ swz_b(k).
__device__ __forceinline__ int swz_a(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz_b(int k) { return ((k >> 2) & 3) << 2; }

template <int TN>
__global__ void __launch_bounds__(kT)
bmm32_kernel(const GemmParams p, int tiles_n) {
  constexpr int kSlot = (kTile + TN) * kBK;  // floats per ring slot: A 128 x 32, then B 32 x TN
  constexpr int NI = TN / 32;                // 16-wide column tiles per wave
  constexpr int CPR = TN / 4;                // 16-byte chunks per B row
  constexpr int BI = kBK * TN / 256 / 4;     // 1 KB B copies per wave per K tile
  constexpr int kStageLd = TN + 4;           // epilogue staging row stride (floats)
  static_assert(kTile * kStageLd <= kRing * kSlot, "the epilogue staging fits in the ring");
  __shared__ __attribute__((aligned(16))) float ring[kRing * kSlot];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int bt = blockIdx.y;
  const bool seg2 = bt >= p.batch_split;
  const int64_t sb = seg2 ? bt - p.batch_split : bt;
  const float* A = static_cast<const float*>(seg2 ? p.A2 : p.A) + sb * p.sA;
  const float* Bm = static_cast<const float*>(seg2 ? p.B2 : p.B) + sb * p.sB;
  const void* Dv = seg2 ? p.D2 : p.D;
  const float* D = Dv ? static_cast<const float*>(Dv) + sb * p.sD : nullptr;
  float* C = static_cast<float*>(seg2 ? p.C2 : p.C) + sb * p.sC;
  void* Cav = seg2 ? p.C2_act : p.C_act;
  bf16_t* Ca = Cav ? static_cast<bf16_t*>(Cav) + sb * p.sC : nullptr;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int m0 = tm * kTile, n0 = tn * TN;
  const int nk = p.K / kBK;

  // K tile t into ring slot t % 4: sixteen 1 KB copies of the A tile (four
  // per wave) and TN / 8 of the B tile (BI per wave)
  auto issue = [&](int t) {
    float* slot = ring + (t & 3) * kSlot;
    const int k0 = t * kBK;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 4 * wave + q;
      const int r = 8 * i + (lane >> 3), cl = lane & 7;
      dma16(A + (int64_t)(m0 + r) * p.lda + k0 + 4 * (cl ^ swz_a(r)),
            reinterpret_cast<const bf16_t*>(slot + 256 * i));
    }
#pragma unroll
    for (int q = 0; q < BI; ++q) {
      const int i = BI * wave + q;
      const int k = (64 / CPR) * i + lane / CPR, cl = lane % CPR;
      dma16(Bm + (int64_t)(k0 + k) * p.ldb + n0 + 4 * (cl ^ swz_b(k)),
            reinterpret_cast<const bf16_t*>(slot + kTile * kBK + 256 * i));
    }
  };

  floatx4 acc[4][NI];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = floatx4{0.f, 0.f, 0.f, 0.f};

  issue(0);
  if (nk > 1) issue(1);
  if (nk > 2) issue(2);
  for (int t = 0; t < nk; ++t) {
    // this wave's copies of tile t landed (tiles t+1, t+2 may be in flight);
    // after the barrier every wave's have, and every wave is done with slot
    // (t - 1) % 4, which tile t + 3 then refills
    if (t + 2 < nk) wait_vm<2 * (4 + BI)>();
    else if (t + 1 < nk) wait_vm<4 + BI>();
    else wait_vm<0>();
    barrier_nofence();
    if (t + 3 < nk) issue(t + 3);
    const float* sA = ring + (t & 3) * kSlot;
    const float* sB = sA + kTile * kBK;
    // the fragments of both 16-deep k groups of the tile: group 1's reads are
    // issued before group 0's products, so only group 0's wait is exposed
    float4 av[2][4];
    float bv[2][4][NI];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int r = 64 * wm + 16 * mi + (lane & 15);
        const int c = 4 * g + (lane >> 4);
        av[g][mi] = *reinterpret_cast<const float4*>(sA + r * kBK + 4 * (c ^ swz_a(r)));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = 16 * g + 4 * (lane >> 4) + j;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int n = (TN / 2) * wn + 16 * ni + (lane & 15);
          bv[g][j][ni] = sB[k * TN + 4 * ((n >> 2) ^ swz_b(k)) + (n & 3)];
        }
      }
    }
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const float4 a4 = av[g][mi];
          const float a = j == 0 ? a4.x : j == 1 ? a4.y : j == 2 ? a4.z : a4.w;
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv[g][j][ni], acc[mi][ni], 0, 0, 0);
        }
  }

  // accumulators -> LDS (row-major) -> 16-byte row pieces with alpha and
  // beta D applied on the way out
  __syncthreads();
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        ring[(64 * wm + 16 * mi + 4 * (lane >> 4) + e) * kStageLd + (TN / 2) * wn + 16 * ni +
             (lane & 15)] = acc[mi][ni][e];
  __syncthreads();
#pragma unroll 4
  for (int q = tid; q < kTile * TN / 4; q += kT) {
    const int r = q / (TN / 4), c4 = 4 * (q % (TN / 4));
    float4 v = *reinterpret_cast<const float4*>(ring + r * kStageLd + c4);
    v.x *= p.alpha; v.y *= p.alpha; v.z *= p.alpha; v.w *= p.alpha;
    if (D) {
      const float4 d = *reinterpret_cast<const float4*>(D + (int64_t)(m0 + r) * p.ldd + n0 + c4);
      v.x += p.beta * d.x; v.y += p.beta * d.y; v.z += p.beta * d.z; v.w += p.beta * d.w;
    }
    const int64_t off = (int64_t)(m0 + r) * p.ldc + n0 + c4;
    *reinterpret_cast<float4*>(C + off) = v;
    if (Ca) {
      union { uint2 u; bf16_t h[4]; } o;
      o.h[0] = f32_to_bf16(v.x); o.h[1] = f32_to_bf16(v.y);
      o.h[2] = f32_to_bf16(v.z); o.h[3] = f32_to_bf16(v.w);
      *reinterpret_cast<uint2*>(Ca + off) = o.u;
    }
  }
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

}  // namespace

bool bmm32_supported(const GemmParams& p, bool a_kmajor, bool b_kmajor) {
  if (!a_kmajor || b_kmajor || p.d_trans || p.ksplit != 1) return false;
  if (p.M != p.N || p.N != p.K || p.M_last != p.M || p.N_last != p.N || p.K_last != p.K) return false;
  if (p.M % kTile != 0 || p.M <= 0) return false;
  const int64_t lds[] = {p.lda, p.ldb, p.ldc, p.ldd, p.sA, p.sB, p.sC, p.sD};
  for (int64_t v : lds)
    if (v % 4 != 0) return false;
  if (p.lda < p.K || p.ldb < p.N || p.ldc < p.N || (p.D && p.ldd < p.N)) return false;
  const bool two = p.batch > p.batch_split;
  const void* ptrs[] = {p.A, p.B, p.C, p.D, two ? p.A2 : nullptr, two ? p.B2 : nullptr,
                        two ? p.C2 : nullptr, two ? p.D2 : nullptr};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return false;
  // bf16 copies are written 8 bytes at a time
  const void* acts[] = {p.C_act, two ? p.C2_act : nullptr};
  for (const void* q : acts)
    if (q && (reinterpret_cast<uintptr_t>(q) & 7u) != 0) return false;
  if (two && (!p.A2 || !p.B2 || !p.C2 || (p.D != nullptr) != (p.D2 != nullptr))) return false;
  return p.batch >= 1 && p.batch <= 65535;
}

hipError_t launch_bmm32(const GemmParams& p, hipStream_t stream) {
  const int tiles_m = p.M / kTile;
  // 128-wide tiles when they fill at least three rounds of one workgroup per
  // CU (256 CUs), else 64-wide ones (twice the workgroups)
  if ((int64_t)tiles_m * tiles_m * p.batch >= 3 * 256) {
    hipLaunchKernelGGL(bmm32_kernel<128>, dim3(tiles_m * tiles_m, p.batch), dim3(kT), 0, stream, p,
                       tiles_m);
  } else {
    hipLaunchKernelGGL(bmm32_kernel<64>, dim3(tiles_m * 2 * tiles_m, p.batch), dim3(kT), 0, stream,
                       p, 2 * tiles_m);
  }
  return hipGetLastError();
}

}  // namespace poetx
