// The backward's gradient apply and gram for 256 x 256 blocks in one pass,
// one workgroup per (block, token range) holding the whole block:
//   Y[t, kb + n] = sum_k X[t, kb + k] M_k[k][n]         (g_Z = g_Y R, g_X = g_U P)
//   part[s][k][i][j] = sum_{t in split s} X[t, kb + i] C[t, kb + j]
//                                                       (G_R = g_Y^T Z, G_P = g_U^T X)
// i.e. the batch-parallel block products of the POET-X layer's backward
// (gist.science technical summary of "POET-X: Memory-efficient LLM Training
// by Scaling Orthogonal Transformation", section 2 Methodik, block-diagonal
// item; the backward is the chain rule of the input-centric forward).
//
// Both products stream X, so one workgroup reads each X tile once for both
// and every operand crosses the CU once. Two workgroups per block, each
// holding one 128-column slab of the block and half of the gram, would each
// have to read all 256 columns of X: twice the bytes through the CU's memory
// pipeline, which bounds these HBM-bound stages.
//
// Four waves, one per SIMD. Wave w keeps columns 64 w .. 64 w + 63 of M_k in
// registers as 32 MFMA B fragments (128 VGPRs) and owns the 128 x 128 quarter
// (w & 1, w >> 1) of the 256 x 256 gram, 16 accumulator tiles of
// v_mfma_f32_32x32x16_bf16 in AGPRs (256). The products are inline asm with
// the gram tied to AGPR operands: with the compiler's builtin, this register
// demand (about 480 per lane) spilled hundreds of VGPRs. The compiler does
// not see the asm products, so the wait states before VALU or memory
// instructions read their results are explicit (s_nop), and the first
// product of each accumulator uses a zero addend instead of a VALU clear.
// Back-to-back products into the same accumulator are interlocked by the
// hardware.
//
// Token tiles of 32 rows of X (32 x 256) and C (32 x 256) go global -> LDS
// with global_load_lds_dwordx4 into a 4-slot ring, three tiles in flight;
// waits are explicit vmcnt counts of this wave's later loads (stores only add
// to the counter, so the waits hold whatever order they complete in). The gram
// reads both tiles with the transposing ds_read_b64_tr_b16; the apply reads
// X's tile as token-major fragments, and its output goes through a staging
// buffer and leaves as 16-byte stores spread over the next tile's products.
// Every element of C is read by the one workgroup that writes Y at the same
// place (the same block columns and tokens), before it writes it, so C and Y
// may be one buffer when Y is row-major. Y may instead be written in the
// tiled layout (kernels.h) for the dense kernel that reads it next; its
// 16-byte pieces then land 64-byte row pieces of 16 KB blocks, and the two
// halves of each 128-byte line come from neighbouring tokens of one store.
#include "common.h"
#include "kernels.h"

namespace poetx {
namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int B = 256;             // block size
constexpr int TT = 32;             // tokens per tile
constexpr int NT = 256;            // threads: four waves
constexpr int XT = TT * B;         // bf16 elements of one operand tile (16 KB)
constexpr int SLOT = 2 * XT;       // X tile, then C tile
constexpr int LPX = XT * 2 / 1024 / 4;  // 1 KB loads per wave per operand tile
constexpr int LPT = 2 * LPX;            // loads per wave per token tile
constexpr int KS = B / 16;         // apply K steps
constexpr int CPT = TT * B / 8 / NT;    // 16-byte output chunks per thread per tile
static_assert(LPT == 8 && CPT == 4 && KS % CPT == 0, "tile shape");

__shared__ __attribute__((aligned(16))) bf16_t g_ga0[SLOT];
__shared__ __attribute__((aligned(16))) bf16_t g_ga1[SLOT];
__shared__ __attribute__((aligned(16))) bf16_t g_ga2[SLOT];
__shared__ __attribute__((aligned(16))) bf16_t g_ga3[SLOT];
__shared__ __attribute__((aligned(16))) bf16_t g_gaout[XT];  // staged Y tile

template <int S> __device__ __forceinline__ bf16_t* ring() {
  return S == 0 ? g_ga0 : S == 1 ? g_ga1 : S == 2 ? g_ga2 : g_ga3;
}
__device__ __forceinline__ bf16_t* ring_rt(int s) {
  return s == 0 ? g_ga0 : s == 1 ? g_ga1 : s == 2 ? g_ga2 : g_ga3;
}

// element offset of (row, col) in a row-major [row][B] tile, 16-byte chunks
// XOR-swizzled by the low 4 row bits
__device__ __forceinline__ int sw(int row, int col) {
  return row * B + ((((col >> 3) ^ (row & 15))) << 3) + (col & 7);
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
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14)); }

struct GramApply {
  const bf16_t* X;
  const bf16_t* C;
  bf16_t* Y;
  int64_t d, col0;
  bool y_tiled;            // Y in the tiled layout (kernels.h)
  int t_begin, t_end, ntiles;
  int tid, lane, wave, wm, wn;
  bf16x8_t bfr[2][KS];     // M_k columns 64 w + 32 j + l % 32, k = 16 ks + 8 (l / 32) ..
  floatx16 gacc[4][4];     // gram quarter (wm, wn), AGPRs

  __device__ __forceinline__ void load_tile(int tile, bf16_t* dst) {
    const int t0 = t_begin + tile * TT;
#pragma unroll
    for (int q = 0; q < LPX; ++q) {
      const int Q = wave * LPX + q;        // 1 KB piece: rows 2 Q, 2 Q + 1
      const int e = Q * 512 + lane * 8;
      const int row = e / B, pch = (e % B) >> 3;
      const int lch = pch ^ (row & 15);
      const int grow = min(t0 + row, t_end - 1);  // rows past the end read a valid row
      dma16(X + (int64_t)grow * d + col0 + lch * 8, dst + Q * 512);
      dma16(C + (int64_t)grow * d + col0 + lch * 8, dst + XT + Q * 512);
    }
  }

  // 32 features (m0 + l % 32) x 8 tokens (k0 + 8 (l / 32) ..) of a
  // token-major tile: the MFMA operand layout, two transposing reads
  __device__ __forceinline__ bf16x8_t gfrag(const bf16_t* tl, int m0, int k0, int ln) const {
    const int g = ln >> 4, i = ln & 15;
    const int m = m0 + 16 * (g & 1) + 4 * (i & 3);
    short4_t h[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int kk = k0 + 8 * (g >> 1) + 4 * hh + (i >> 2);
      h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(tl + sw(kk, m)));
    }
    union { short4_t s[2]; bf16x8_t v; } u;
    u.s[0] = h[0];
    u.s[1] = h[1];
    return u.v;
  }

  template <int I, int J, bool ZERO>
  __device__ __forceinline__ void gmma(const bf16x8_t& a, const bf16x8_t& c) {
    if (ZERO)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=a"(gacc[I][J]) : "v"(a), "v"(c));
    else
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(gacc[I][J]) : "v"(a), "v"(c));
  }

  // the gram's 16 tokens k0 .. k0 + 15 of the tile in slot st
  template <bool ZERO>
  __device__ __forceinline__ void gram_step(const bf16_t* st, int k0, int ln) {
    bf16x8_t fa[4], fc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = gfrag(st, wm * 128 + 32 * i, k0, ln);
#pragma unroll
    for (int j = 0; j < 4; ++j) fc[j] = gfrag(st + XT, wn * 128 + 32 * j, k0, ln);
    gmma<0, 0, ZERO>(fa[0], fc[0]); gmma<0, 1, ZERO>(fa[0], fc[1]);
    gmma<0, 2, ZERO>(fa[0], fc[2]); gmma<0, 3, ZERO>(fa[0], fc[3]);
    gmma<1, 0, ZERO>(fa[1], fc[0]); gmma<1, 1, ZERO>(fa[1], fc[1]);
    gmma<1, 2, ZERO>(fa[1], fc[2]); gmma<1, 3, ZERO>(fa[1], fc[3]);
    gmma<2, 0, ZERO>(fa[2], fc[0]); gmma<2, 1, ZERO>(fa[2], fc[1]);
    gmma<2, 2, ZERO>(fa[2], fc[2]); gmma<2, 3, ZERO>(fa[2], fc[3]);
    gmma<3, 0, ZERO>(fa[3], fc[0]); gmma<3, 1, ZERO>(fa[3], fc[1]);
    gmma<3, 2, ZERO>(fa[3], fc[2]); gmma<3, 3, ZERO>(fa[3], fc[3]);
  }

  // output chunk q of the staged tile whose first token is t0
  __device__ __forceinline__ void store_chunk(int q, int t0, int td) {
    const int c = td + q * NT;
    const int row = c / (B / 8), ch = c % (B / 8);
    const uint4 v = *reinterpret_cast<const uint4*>(g_gaout + sw(row, ch * 8));
    if (t0 + row < t_end) {
      const int64_t off = y_tiled ? tiled_offset(t0 + row, col0 + ch * 8, d)
                                  : (int64_t)(t0 + row) * d + col0 + ch * 8;
      *reinterpret_cast<uint4*>(Y + off) = v;
    }
  }

  template <int S, bool FIRST>
  __device__ __forceinline__ void tile(int t) {
    bf16_t* st = ring<S>();
    // opaque copies of the lane and thread ids: keeps the compiler from
    // hoisting this tile's address arithmetic out of the loop
    int ln = lane, td = tid;
    asm volatile("" : "+v"(ln), "+v"(td));
    if (t + 2 < ntiles) wait_vm<2 * LPT>();
    else if (t + 1 < ntiles) wait_vm<LPT>();
    else wait_vm<0>();
    wait_lds();  // this wave's staging writes of tile t-1 landed
    __builtin_amdgcn_s_barrier();  // every wave's part of tile t landed; slot of t-1 free
    if (t + 3 < ntiles) load_tile(t + 3, ring<(S + 3) & 3>());

    const int valid = t_end - (t_begin + t * TT);
    if (valid < TT) {
      // ragged last tile: rows past the end repeat a valid token; zero them in
      // X's tile so they add nothing to the gram (their outputs are not stored)
      for (int e = td; e < (TT - valid) * B; e += NT) st[sw(valid + e / B, e % B)] = 0;
      __syncthreads();
    }
    gram_step<FIRST>(st, 0, ln);
    gram_step<false>(st, 16, ln);

    // apply: 32 tokens x this wave's 64 output columns; the product's first
    // operand is the block, so acc[j] holds Y^T
    floatx16 acc[2];
    bf16x8_t af[2];
    auto rd = [&](int ks, bf16x8_t& a) {
      a = *reinterpret_cast<const bf16x8_t*>(st + sw(ln & 31, 16 * ks + 8 * (ln >> 5)));
    };
    rd(0, af[0]);
    const int tp0 = t_begin + (t - 1) * TT;  // first token of the staged tile t-1
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) rd(ks + 1, af[(ks + 1) & 1]);
      if (t > 0 && ks % (KS / CPT) == 0) store_chunk(ks / (KS / CPT), tp0, td);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (ks == 0)
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                       : "=v"(acc[j]) : "v"(bfr[j][ks]), "v"(af[ks & 1]));
        else
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                       : "+v"(acc[j]) : "v"(bfr[j][ks]), "v"(af[ks & 1]));
      }
    }
    // wait states before VALU reads of the products' results (the sched
    // barriers keep those reads behind them)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();  // all waves done reading slot S and the staged tile t-1
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // lane l has token l % 32 and, for e = 4 g .. 4 g + 3, the four
      // consecutive columns 64 w + 32 j + 8 g + 4 (l / 32) + (e % 4)
      const int m = ln & 31;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = 64 * wave + 32 * j + 8 * g + 4 * (ln >> 5);
        short4_t v;
        v[0] = (short)f32_to_bf16(acc[j][4 * g + 0]);
        v[1] = (short)f32_to_bf16(acc[j][4 * g + 1]);
        v[2] = (short)f32_to_bf16(acc[j][4 * g + 2]);
        v[3] = (short)f32_to_bf16(acc[j][4 * g + 3]);
        *reinterpret_cast<short4_t*>(g_gaout + sw(m, n)) = v;
      }
    }
    // no barrier: the next tile's first barrier orders these writes before
    // its reads of the staging buffer
  }
};

// Workgroup unit = split * nb + blk (one round: nb * nsplit <= 256).
__global__ void __launch_bounds__(NT)
gramapply256_kernel(const bf16_t* __restrict__ X, const bf16_t* __restrict__ Mb, bf16_t* Y,
                    int tokens, int64_t d, int nb, int nsplit, int tok_per_wg, const bf16_t* C,
                    float* __restrict__ part, int y_tiled) {
  GramApply k;
  k.tid = threadIdx.x;
  k.lane = k.tid & 63;
  k.wave = __builtin_amdgcn_readfirstlane(k.tid >> 6);
  k.wm = k.wave & 1;
  k.wn = k.wave >> 1;
  const int unit = blockIdx.x;
  if (unit >= nb * nsplit) return;
  const int blk = unit % nb;
  const int split = unit / nb;
  k.t_begin = split * tok_per_wg;
  k.t_end = min(tokens, k.t_begin + tok_per_wg);
  if (k.t_begin >= k.t_end) return;
  k.X = X;
  k.C = C;
  k.Y = Y;
  k.y_tiled = y_tiled != 0;
  k.d = d;
  k.col0 = (int64_t)blk * B;
  k.ntiles = (k.t_end - k.t_begin + TT - 1) / TT;

  // B(n, k) = M[k][n]: all 256 rows of M_k go to LDS (64 rows per ring
  // slot), and each fragment (8 consecutive k of column n) comes back with
  // two transposing reads of 4 k each
  {
    const bf16_t* src0 = Mb + (int64_t)blk * B * B;
    constexpr int ROWS = SLOT / B;  // rows per slot
    for (int c = k.tid; c < B * B / 8; c += NT) {
      const int row = c / (B / 8), ch = c % (B / 8);
      *reinterpret_cast<uint4*>(ring_rt(row / ROWS) + sw(row % ROWS, ch * 8)) =
          *reinterpret_cast<const uint4*>(src0 + (int64_t)row * B + ch * 8);
    }
    __syncthreads();
    const int lane = k.lane;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int g = lane >> 4, i = lane & 15;
        const int n = 64 * k.wave + 32 * j + 16 * (g & 1) + 4 * (i & 3);
        short4_t h[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int kk = 16 * ks + 8 * (g >> 1) + 4 * hh + (i >> 2);
          h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_short4*)(ring_rt(kk / ROWS) + sw(kk % ROWS, n)));
        }
        union { short4_t s[2]; bf16x8_t v; } u;
        u.s[0] = h[0];
        u.s[1] = h[1];
        k.bfr[j][ks] = u.v;
      }
    __syncthreads();  // the ring is reused for token tiles
  }

  const int nt = k.ntiles;
  k.load_tile(0, ring<0>());
  if (nt > 1) k.load_tile(1, ring<1>());
  if (nt > 2) k.load_tile(2, ring<2>());
  k.tile<0, true>(0);
  int t = 1;
  for (; t + 4 <= nt; t += 4) {
    k.tile<1, false>(t);
    k.tile<2, false>(t + 1);
    k.tile<3, false>(t + 2);
    k.tile<0, false>(t + 3);
  }
  if (t < nt) k.tile<1, false>(t++);
  if (t < nt) k.tile<2, false>(t++);
  if (t < nt) k.tile<3, false>(t++);
  __syncthreads();  // the last tile is staged
#pragma unroll
  for (int q = 0; q < CPT; ++q) k.store_chunk(q, k.t_begin + (nt - 1) * TT, k.tid);
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  // gram quarter: lane l of tile (i, j) holds rows 8 (e / 4) + 4 (l / 32) + e % 4
  // of the 32-row block and column l % 32
  float* out = part + ((int64_t)split * nb + blk) * B * B;
  const int lane = k.lane;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = k.wn * 128 + 32 * j + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = k.wm * 128 + 32 * i + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        out[(int64_t)m * B + n] = k.gacc[i][j][e];
      }
    }
}

}  // namespace

hipError_t launch_gramapply256(const void* X, const void* M, const void* C, void* Y, float* part,
                               int64_t tokens, int64_t d, int max_split, int* nsplit, bool y_tiled,
                               hipStream_t s) {
  if (d % B != 0 || tokens < 1 || max_split < 1) return hipErrorInvalidValue;
  if (y_tiled && (tokens % kTileRows != 0 || C == Y)) return hipErrorInvalidValue;
  const int nb = (int)(d / B);
  // one round of at most 256 workgroups, whole tiles per split, and no more
  // splits than the caller's partial buffer holds
  int splits = 256 / nb;
  const int max_tiles = (int)((tokens + TT - 1) / TT);
  if (splits > max_tiles) splits = max_tiles;
  if (splits > max_split) splits = max_split;
  if (splits < 1) splits = 1;
  int per = (int)((tokens + splits - 1) / splits);
  per = (per + TT - 1) / TT * TT;
  splits = (int)((tokens + per - 1) / per);  // every split holds at least one token
  hipLaunchKernelGGL(gramapply256_kernel, dim3(nb * splits), dim3(NT), 0, s,
                     static_cast<const bf16_t*>(X), static_cast<const bf16_t*>(M),
                     static_cast<bf16_t*>(Y), (int)tokens, d, nb, splits, per,
                     static_cast<const bf16_t*>(C), part, (int)y_tiled);
  *nsplit = splits;
  return hipGetLastError();
}

}  // namespace poetx
