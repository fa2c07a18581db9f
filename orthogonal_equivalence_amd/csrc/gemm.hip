// Batched split-K GEMM on CDNA4 matrix cores (MFMA), used for every
// contraction of the POET-X layer: the block-diagonal applies of R and P
// (batched over blocks), the dense W0 products, the token-reduction grams
// G_R and G_P (split over tokens), and the Cayley VJP products.
//
// One workgroup computes a BM x BN tile of one batch (and one K split). Both
// operand tiles are staged in LDS K-contiguous ([rows][BK + pad]) in two
// buffers: the next tile's global loads are issued before the MFMAs on the
// current one, and one barrier per K step separates the LDS write of the
// next buffer from the reads of the current one. An operand that is
// contiguous along M/N in global memory (a transposed access, e.g. the
// token-major activations of the grams) is loaded as VEC x VEC sub-blocks of
// 16-byte rows and transposed in registers on the way to LDS.
//
// bf16 inputs use v_mfma_f32_16x16x32_bf16, float32 inputs
// v_mfma_f32_16x16x4_f32; accumulation is float32 in both cases.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace poetx {
namespace {

template <typename T>
struct Vec16 {  // 16 bytes of T
  static constexpr int N = ElemTraits<T>::kVec;
  union {
    uint4 u;
    T e[N];
  };
};

template <typename TIn, int ROWS, int BK, int NT, bool KMAJ>
struct TileLoader {
  static constexpr int VEC = ElemTraits<TIn>::kVec;
  static constexpr int LDK = BK + VEC;
  // K-major: one 16-byte chunk (VEC consecutive k of one row) per item.
  // MN-major: one VEC(k) x VEC(row) sub-block per item.
  static constexpr int ITEMS = KMAJ ? ROWS * BK / VEC : (ROWS / VEC) * (BK / VEC);
  static constexpr int PER_THREAD = (ITEMS + NT - 1) / NT;
  static constexpr int REGS = KMAJ ? PER_THREAD : PER_THREAD * VEC;

  Vec16<TIn> r[REGS];

  // base points at element (row 0, k 0) of this batch; rows/k are global
  // indices. Rows >= rext or k >= kend read as zero.
  __device__ __forceinline__ void load(const TIn* __restrict__ base, int64_t ld, int r0, int rext,
                                       int k0, int kend, int tid) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int item = tid + i * NT;
      if (KMAJ) {
        Vec16<TIn>& v = r[i];
        v.u = make_uint4(0, 0, 0, 0);
        if (item < ITEMS) {
          const int row = item / (BK / VEC);
          const int kc = (item % (BK / VEC)) * VEC;
          const int gr = r0 + row, gk = k0 + kc;
          if (gr < rext && gk < kend) {
            const TIn* src = base + (int64_t)gr * ld + gk;
            if (gk + VEC <= kend) {
              v.u = *reinterpret_cast<const uint4*>(src);
            } else {
#pragma unroll
              for (int e = 0; e < VEC; ++e)
                if (gk + e < kend) v.e[e] = src[e];
            }
          }
        }
      } else {
        const int kb = item / (ROWS / VEC);
        const int rb = item % (ROWS / VEC);
        const int gr = r0 + rb * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          Vec16<TIn>& v = r[i * VEC + e];
          v.u = make_uint4(0, 0, 0, 0);
          const int gk = k0 + kb * VEC + e;
          if (item < ITEMS && gr < rext && gk < kend)
            v.u = *reinterpret_cast<const uint4*>(base + (int64_t)gk * ld + gr);
        }
      }
    }
  }

  __device__ __forceinline__ void store(TIn* __restrict__ s, int tid) const {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int item = tid + i * NT;
      if (item >= ITEMS) continue;
      if (KMAJ) {
        const int row = item / (BK / VEC);
        const int kc = (item % (BK / VEC)) * VEC;
        *reinterpret_cast<uint4*>(s + row * LDK + kc) = r[i].u;
      } else {
        const int kb = item / (ROWS / VEC);
        const int rb = item % (ROWS / VEC);
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
          Vec16<TIn> t;
#pragma unroll
          for (int e = 0; e < VEC; ++e) t.e[e] = r[i * VEC + e].e[c];
          *reinterpret_cast<uint4*>(s + (rb * VEC + c) * LDK + kb * VEC) = t.u;
        }
      }
    }
  }
};

template <typename TIn> struct Mfma;

template <> struct Mfma<bf16_t> {
  static constexpr int KSTEP = 32;
  typedef bf16x8_t Frag;
  __device__ static Frag load(const bf16_t* s, int LDK, int row, int kk, int lane) {
    return *reinterpret_cast<const bf16x8_t*>(s + (row + (lane & 15)) * LDK + kk + 8 * (lane >> 4));
  }
  __device__ static floatx4 mma(Frag a, Frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int KSTEP = 4;
  typedef float Frag;
  __device__ static Frag load(const float* s, int LDK, int row, int kk, int lane) {
    return s[(row + (lane & 15)) * LDK + kk + (lane >> 4)];
  }
  __device__ static floatx4 mma(Frag a, Frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

template <typename TIn, typename TOut, bool A_KMAJ, bool B_KMAJ, int BM, int BN, int BK, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_kernel(const GemmParams p) {
  constexpr int NT = 64 * WM * WN;
  constexpr int VEC = ElemTraits<TIn>::kVec;
  constexpr int LDK = BK + VEC;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int STAGE = (BM + BN) * LDK;
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(BK % Mfma<TIn>::KSTEP == 0 && BK % VEC == 0, "bad K tile");

  __shared__ __attribute__((aligned(16))) TIn smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;

  const int bt = blockIdx.y;
  const bool last = (bt == p.batch - 1);
  const int Mx = last ? p.M_last : p.M;
  const int Nx = last ? p.N_last : p.N;
  const int Kx = last ? p.K_last : p.K;
  const int num_mt = (p.M + BM - 1) / BM;
  const int m0 = (blockIdx.x % num_mt) * BM;
  const int n0 = (blockIdx.x / num_mt) * BN;
  if (m0 >= Mx || n0 >= Nx) return;  // whole workgroup: tile outside a ragged last batch

  const int kbeg = blockIdx.z * p.kchunk;
  const int kend = min(Kx, kbeg + p.kchunk);
  const int ntiles = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

  const TIn* A = static_cast<const TIn*>(p.A) + (int64_t)bt * p.sA;
  const TIn* B = static_cast<const TIn*>(p.B) + (int64_t)bt * p.sB;

  TileLoader<TIn, BM, BK, NT, A_KMAJ> la;
  TileLoader<TIn, BN, BK, NT, B_KMAJ> lb;

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  if (ntiles > 0) {
    la.load(A, p.lda, m0, Mx, kbeg, kend, tid);
    lb.load(B, p.ldb, n0, Nx, kbeg, kend, tid);
    la.store(smem, tid);
    lb.store(smem + BM * LDK, tid);
    __syncthreads();
  }

  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    const bool more = (t + 1) < ntiles;
    if (more) {
      const int k0 = kbeg + (t + 1) * BK;
      la.load(A, p.lda, m0, Mx, k0, kend, tid);
      lb.load(B, p.ldb, n0, Nx, k0, kend, tid);
    }
    const TIn* As = smem + cur * STAGE;
    const TIn* Bs = As + BM * LDK;
#pragma unroll
    for (int kk = 0; kk < BK; kk += Mfma<TIn>::KSTEP) {
      typename Mfma<TIn>::Frag af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = Mfma<TIn>::load(As, LDK, wm * TM + i * 16, kk, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = Mfma<TIn>::load(Bs, LDK, wn * TN + j * 16, kk, lane);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = Mfma<TIn>::mma(af[i], bfr[j], acc[i][j]);
    }
    if (more) {
      TIn* nxt = smem + (cur ^ 1) * STAGE;
      la.store(nxt, tid);
      lb.store(nxt + BM * LDK, tid);
    }
    __syncthreads();
  }

  TOut* C = static_cast<TOut*>(p.C) + (int64_t)bt * p.sC + (int64_t)blockIdx.z * p.sC_split;
  const TOut* D = p.D ? static_cast<const TOut*>(p.D) + (int64_t)bt * p.sD : nullptr;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * TN + j * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * TM + i * 16 + 4 * (lane >> 4) + e;
        if (m < Mx && n < Nx) {
          float v = p.alpha * acc[i][j][e];
          if (D) v += p.beta * ElemTraits<TOut>::to_f32(D[(int64_t)m * p.ldd + n]);
          store_as<TOut>(C + (int64_t)m * p.ldc + n, v);
        }
      }
    }
  }
}

// Tile shapes: bf16 128 x 128 x 64 with 2 x 2 waves (64 x 64 per wave);
// float32 64 x 64 x 32 with 2 x 2 waves (32 x 32 per wave).
template <typename TIn> struct TileCfg;
template <> struct TileCfg<bf16_t> { static constexpr int BM = 128, BN = 128, BK = 64, WM = 2, WN = 2; };
template <> struct TileCfg<float> { static constexpr int BM = 64, BN = 64, BK = 32, WM = 2, WN = 2; };

template <typename TIn, typename TOut, bool AK, bool BK_>
hipError_t launch_cfg(const GemmParams& p, hipStream_t stream) {
  typedef TileCfg<TIn> C;
  const int num_mt = (p.M + C::BM - 1) / C::BM;
  const int num_nt = (p.N + C::BN - 1) / C::BN;
  dim3 grid(num_mt * num_nt, p.batch, p.ksplit);
  dim3 block(64 * C::WM * C::WN);
  hipLaunchKernelGGL((gemm_kernel<TIn, TOut, AK, BK_, C::BM, C::BN, C::BK, C::WM, C::WN>), grid, block,
                     0, stream, p);
  return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_layout(bool ak, bool bk, const GemmParams& p, hipStream_t stream) {
  if (ak && bk) return launch_cfg<TIn, TOut, true, true>(p, stream);
  if (ak && !bk) return launch_cfg<TIn, TOut, true, false>(p, stream);
  if (!ak && !bk) return launch_cfg<TIn, TOut, false, false>(p, stream);
  return launch_cfg<TIn, TOut, false, true>(p, stream);
}

}  // namespace

int gemm_k_tile(DType in) { return in == DType::BF16 ? TileCfg<bf16_t>::BK : TileCfg<float>::BK; }

hipError_t launch_gemm(DType in, DType out, bool a_kmajor, bool b_kmajor, const GemmParams& p,
                       hipStream_t stream) {
  if (p.batch <= 0 || p.M <= 0 || p.N <= 0 || p.ksplit <= 0) return hipSuccess;
  if (in == DType::BF16) {
    if (out == DType::BF16) return launch_layout<bf16_t, bf16_t>(a_kmajor, b_kmajor, p, stream);
    return launch_layout<bf16_t, float>(a_kmajor, b_kmajor, p, stream);
  }
  if (out == DType::F32) return launch_layout<float, float>(a_kmajor, b_kmajor, p, stream);
  return hipErrorInvalidValue;
}

}  // namespace poetx
