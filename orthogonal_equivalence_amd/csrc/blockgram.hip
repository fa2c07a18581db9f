// Streaming token-reduction grams of the POET-X backward: for every block k
// of b features (b = 128, 256 or 512) and a range of tokens,
//   part[s][k] = sum_{t in split s} A[t, kb:kb+b]^T C[t, kb:kb+b]   (fp32, b x b)
// which gives dL/dR_k = g_Y[:, k]^T Z[:, k] and dL/dP_j = g_U[:, j]^T X[:, j]
// (chain rule of the block-diagonal products; gist.science technical summary
// of "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
// Transformation", section 2 Methodik, block-diagonal item).
//
// One workgroup owns one block (b = 512: one 256 x 256 quadrant of it) and
// one token range and keeps that b x b (256 x 256) result in accumulators (a
// 2 x 2 wave grid, v_mfma_f32_32x32x16_bf16). The four quadrant workgroups of
// a 512 block and token range are launched 8 workgroup ids apart, so they run
// on one XCD at about the same time and each 256-column half of A and C
// streamed by two of them is read from HBM about once. Both
// operands are token-major, so the MFMA fragments (8 consecutive tokens for a
// fixed feature) are read from the row-major LDS tiles with the gfx950
// transposing read ds_read_b64_tr_b16. Token tiles of 32 rows of both inputs
// are copied straight into a 4-stage LDS ring (global_load_lds_dwordx4, three
// tiles in flight, explicit waits as in the block apply).
#include "common.h"
#include "kernels.h"

namespace poetx {
namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kTT = 32;    // tokens per tile
constexpr int kNT = 256;
constexpr int kSlot = 2 * kTT * 256;  // bf16 elements per ring slot (A and C tiles, b <= 256)

__shared__ __attribute__((aligned(16))) bf16_t g_gr0[kSlot];
__shared__ __attribute__((aligned(16))) bf16_t g_gr1[kSlot];
__shared__ __attribute__((aligned(16))) bf16_t g_gr2[kSlot];
__shared__ __attribute__((aligned(16))) bf16_t g_gr3[kSlot];

template <int S> __device__ __forceinline__ bf16_t* slot() {
  return S == 0 ? g_gr0 : S == 1 ? g_gr1 : S == 2 ? g_gr2 : g_gr3;
}

// LDS element offset of (row, col) in a row-major [token][feature] tile of
// width W: 16-byte chunk c of row r stored at c ^ 4 (r & 3). For the
// transposing fragment reads below (rows k .. k + 3 and k + 8 .. of 16 or 32
// features) this measured 6 % faster on gfx950 than c ^ (r & 15) (gram_p
// 34.0 -> 32.3 us) with fewer LDS bank conflicts.
template <int W>
__device__ __forceinline__ int sw(int row, int col) {
  return row * W + ((((col >> 3) ^ ((row & 3) << 2))) << 3) + (col & 7);
}

__device__ __forceinline__ void dma16(const void* gptr, const bf16_t* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)lds_base)));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m0), "v"(gptr)
               : "memory", "m0");
}

template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// B: width of the streamed column ranges (and of the workgroup's result)
template <int B>
struct BlockGram {
  static constexpr int WT = B / 2;            // wave tile (2 x 2 waves)
  static constexpr int FB = WT / 32;          // 32-blocks per wave tile side
  static constexpr int TILE = kTT * B;        // elements of one operand tile
  static constexpr int LPW = 2 * TILE * 2 / 1024 / 4;  // 1 KB loads per wave per tile

  const bf16_t* A;  // first column of this workgroup's A range
  const bf16_t* C;  // first column of its C range
  int64_t d;
  int t_begin, t_end, ntiles;
  int lane, wave, wm, wn;
  floatx16 acc[FB][FB];

  __device__ __forceinline__ void load_tile(int tile, bf16_t* dst) {
    const int t0 = t_begin + tile * kTT;
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
      const int Q = wave * LPW + q;               // 1 KB piece: first half A, second half C
      const int half = Q / (LPW * 2);
      const int Qh = Q - half * (LPW * 2);
      const int e = Qh * 512 + lane * 8;
      const int row = e / B, pch = (e % B) >> 3;
      const int lch = pch ^ ((row & 3) << 2);
      const int grow = min(t0 + row, t_end - 1);
      const bf16_t* src = (half == 0 ? A : C) + (int64_t)grow * d + lch * 8;
      dma16(src, dst + half * TILE + Qh * 512);
    }
  }

  // 8 consecutive tokens (k) x 32 features (m) fragment from a [token][feature]
  // tile, read with two transposing loads
  __device__ __forceinline__ bf16x8_t frag(const bf16_t* tile, int m0, int k0) const {
    const int g = lane >> 4, i = lane & 15;
    const int m = m0 + 16 * (g & 1) + 4 * (i & 3);
    short4_t h[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int k = k0 + 8 * (g >> 1) + 4 * hh + (i >> 2);
      h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(tile + sw<B>(k, m)));
    }
    union { short4_t s[2]; bf16x8_t v; } u;
    u.s[0] = h[0];
    u.s[1] = h[1];
    return u.v;
  }

  template <int S>
  __device__ __forceinline__ void tile(int t) {
    if (t + 2 < ntiles) wait_vm<2 * LPW>();
    else if (t + 1 < ntiles) wait_vm<LPW>();
    else wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    if (t + 3 < ntiles) load_tile(t + 3, slot<(S + 3) & 3>());
    bf16_t* tw = slot<S>();
    const int valid = t_end - (t_begin + t * kTT);
    if (valid < kTT) {
      // ragged last tile: rows past the end were loaded from a repeated valid
      // token; zero them in the A tile so they add nothing to the gram
      for (int e = threadIdx.x; e < (kTT - valid) * B; e += kNT) {
        const int row = valid + e / B, col = e % B;
        tw[sw<B>(row, col)] = 0;
      }
      __syncthreads();
    }
    const bf16_t* ta = tw;
    const bf16_t* tc = ta + TILE;
    bf16x8_t fa[2][FB], fc[2][FB];
#pragma unroll
    for (int i = 0; i < FB; ++i) fa[0][i] = frag(ta, wm * WT + 32 * i, 0);
#pragma unroll
    for (int j = 0; j < FB; ++j) fc[0][j] = frag(tc, wn * WT + 32 * j, 0);
#pragma unroll
    for (int ks = 0; ks < kTT / 16; ++ks) {
      if (ks + 1 < kTT / 16) {
#pragma unroll
        for (int i = 0; i < FB; ++i) fa[(ks + 1) & 1][i] = frag(ta, wm * WT + 32 * i, 16 * (ks + 1));
#pragma unroll
        for (int j = 0; j < FB; ++j) fc[(ks + 1) & 1][j] = frag(tc, wn * WT + 32 * j, 16 * (ks + 1));
      }
#pragma unroll
      for (int i = 0; i < FB; ++i)
#pragma unroll
        for (int j = 0; j < FB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks & 1][i], fc[ks & 1][j], acc[i][j], 0, 0, 0);
    }
  }
};

// QS x QS workgroups per block of size QS * B (QS = 1, or 2 for b = 512):
// workgroup (split, blk, p, q) accumulates rows p B.. and columns q B.. of
// part[split][blk] (row stride QS * B) from A's columns p B.. and C's columns
// q B.. of the block.
template <int B, int QS>
__global__ void __launch_bounds__(kNT)
blockgram_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ C, float* __restrict__ part,
                 int tokens, int64_t d, int nb, int nsplit, int tok_per_split) {
  typedef BlockGram<B> K;
  constexpr int BB = QS * B;  // block size
  K k;
  const int tid = threadIdx.x;
  k.lane = tid & 63;
  k.wave = tid >> 6;
  k.wm = k.wave & 1;
  k.wn = k.wave >> 1;
  int unit, quad = 0;
  if (QS == 1) {
    unit = blockIdx.x;
  } else {
    // ids 32 g + 8 quad + r: unit 8 g + r, its four quadrants 8 ids apart
    unit = (int)(blockIdx.x >> 5) * 8 + (int)(blockIdx.x & 7);
    quad = (int)(blockIdx.x >> 3) & 3;
  }
  if (unit >= nb * nsplit) return;  // padding id of the last group (uniform, before any barrier)
  const int blk = unit % nb;
  const int split = unit / nb;
  const int p = quad >> 1, q = quad & 1;
  k.t_begin = split * tok_per_split;
  k.t_end = min(tokens, k.t_begin + tok_per_split);
  k.A = A + (int64_t)blk * BB + p * B;
  k.C = C + (int64_t)blk * BB + q * B;
  k.d = d;
#pragma unroll
  for (int i = 0; i < K::FB; ++i)
#pragma unroll
    for (int j = 0; j < K::FB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) k.acc[i][j][e] = 0.f;
  // a split past the end (never produced by the host) still writes zeros
  k.ntiles = k.t_end > k.t_begin ? (k.t_end - k.t_begin + kTT - 1) / kTT : 0;
  const int nt = k.ntiles;
  if (nt > 0) k.load_tile(0, slot<0>());
  if (nt > 1) k.load_tile(1, slot<1>());
  if (nt > 2) k.load_tile(2, slot<2>());
  int t = 0;
  for (; t + 4 <= nt; t += 4) {
    k.template tile<0>(t);
    k.template tile<1>(t + 1);
    k.template tile<2>(t + 2);
    k.template tile<3>(t + 3);
  }
  if (t < nt) k.template tile<0>(t++);
  if (t < nt) k.template tile<1>(t++);
  if (t < nt) k.template tile<2>(t++);

  float* out = part + ((int64_t)split * nb + blk) * BB * BB + (int64_t)(p * B) * BB + q * B;
  const int lane = k.lane;
#pragma unroll
  for (int i = 0; i < K::FB; ++i)
#pragma unroll
    for (int j = 0; j < K::FB; ++j) {
      const int n = k.wn * K::WT + 32 * j + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = k.wm * K::WT + 32 * i + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        out[(int64_t)m * BB + n] = k.acc[i][j][e];
      }
    }
}

}  // namespace

bool blockgram_supported(DType t, int64_t d, int b) {
  return t == DType::BF16 && (b == 128 || b == 256 || b == 512) && d % b == 0;
}

int blockgram_wg_per_block(int b) { return b == 512 ? 4 : 1; }

hipError_t launch_blockgram(const void* A, const void* C, float* part, int64_t tokens, int64_t d,
                            int b, int nsplit, int kchunk, hipStream_t s) {
  const int nb = (int)(d / b);
  const bf16_t* a = static_cast<const bf16_t*>(A);
  const bf16_t* c = static_cast<const bf16_t*>(C);
  if (b == 512) {
    const int units = nb * nsplit;
    hipLaunchKernelGGL((blockgram_kernel<256, 2>), dim3((units + 7) / 8 * 32), dim3(kNT), 0, s, a, c,
                       part, (int)tokens, d, nb, nsplit, kchunk);
  } else if (b == 256) {
    hipLaunchKernelGGL((blockgram_kernel<256, 1>), dim3(nb * nsplit), dim3(kNT), 0, s, a, c, part,
                       (int)tokens, d, nb, nsplit, kchunk);
  } else {
    hipLaunchKernelGGL((blockgram_kernel<128, 1>), dim3(nb * nsplit), dim3(kNT), 0, s, a, c, part,
                       (int)tokens, d, nb, nsplit, kchunk);
  }
  return hipGetLastError();
}

}  // namespace poetx
