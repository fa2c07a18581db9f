// Streaming block-diagonal apply for bf16 activations: for every block k of
// b features (b = 128, 256 or 512) and every token t,
//   Y[t, kb + n] = sum_k X[t, kb + k] B(n, k),  B(n, k) = M_k[n][k] (transpose)
//                                               or      M_k[k][n],
// i.e. the batch-parallel block products of the POET-X layer (gist.science
// technical summary of "POET-X: Memory-efficient LLM Training by Scaling
// Orthogonal Transformation", section 2 Methodik, block-diagonal item):
// P-apply and R-apply of the forward (transpose) and the gradients through R
// and P of the backward (no transpose).
//
// These products are HBM-bound (about b/2 flop per byte), so the kernel is
// built to stream: one workgroup owns one block and a contiguous token range
// (about one workgroup per CU). It loads M_k once and keeps it in registers
// as MFMA B fragments: wave w owns output columns [w b/4, (w+1) b/4). With the
// transpose a fragment is part of one row of M_k, loaded straight from global
// memory while the first token tiles are in flight; otherwise it is part of a
// column, so M_k goes through LDS and comes back with the gfx950 transposing
// LDS read ds_read_b64_tr_b16. At b = 512 the block (512 KB) does not fit one
// CU's registers: two workgroups share a block and token range, each holding
// the 256 output columns of its slab (512 x 256 bf16, 256 KB: 256 VGPRs per
// lane; through the LDS ring in two passes when staged) and streaming 32-token
// tiles of all 512 input columns; the two are launched 8 workgroup ids apart,
// so they run on one XCD at about the same time and the input tile they both
// read comes from HBM about once. (Four 128-column slabs per block were ~10 %
// slower: each input fragment then fed one MFMA instead of two.)
// Token tiles of 64 rows (b <= 256) are copied from global
// memory straight into a 4-stage LDS ring (global_load_lds_dwordx4, three
// tiles in flight) and multiplied on v_mfma_f32_32x32x16_bf16 with the block
// as the first operand, so the accumulators hold the transposed output tile:
// each lane has four consecutive output columns of one token, which go to an
// output staging buffer as one 8-byte LDS write (not four 2-byte ones). The
// staged tile leaves with 16-byte stores spread over the next tile's products
// (the staging buffer is not a ring slot, so nothing waits for the stores
// before the ring moves on; 5-7 % faster than staging into the consumed slot
// and storing before the next tile). Each tile derives its addresses from an opaque copy of
// the lane id, so none are hoisted out of the tile loop to hold registers
// (322 VGPRs at b = 256, against 509 with the hoisted form).
//
// The backward's gradient apply and gram share their streamed operand (g_Y
// for R, g_U for P), so one launch does both (GRAM): each ring slot also
// carries the tile of C's columns matching the workgroup's output columns,
// and the workgroup accumulates that part of the gram X^T C
// (v_mfma_f32_32x32x16_bf16, fragments read with the transposing LDS read).
// At b = 128 a workgroup holds the whole block and its whole 128 x 128 gram
// (64-token tiles), so every operand crosses the CU once. The b = 256 case,
// whose block and gram need about 480 registers per lane, is its own kernel
// (gramapply.hip).
//
// Waits on the LDS-bound loads are explicit: before tile t, the wave waits
// until at most (number of its tile loads issued after tile t) vector memory
// operations are outstanding. Stores only add to that counter, so the wait is
// correct whatever order loads and stores complete in.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace poetx {
namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kNT = 256;   // threads
constexpr int kStage = 64 * 256;  // bf16 elements per ring slot (a 64 x 256 or 32 x 512 tile)

// The ring slots are separate arrays so that the compiler can tell which slot
// an LDS read touches while loads into the other slots are in flight.
__shared__ __attribute__((aligned(16))) bf16_t g_ring0[kStage];
__shared__ __attribute__((aligned(16))) bf16_t g_ring1[kStage];
__shared__ __attribute__((aligned(16))) bf16_t g_ring2[kStage];
__shared__ __attribute__((aligned(16))) bf16_t g_ring3[kStage];
// output staging: tile t's result (at most 64 x 256) waits here while tile
// t+1's products run; with the ring, 160 KB of LDS
__shared__ __attribute__((aligned(16))) bf16_t g_out[kStage];

template <int S> __device__ __forceinline__ bf16_t* ring() {
  return S == 0 ? g_ring0 : S == 1 ? g_ring1 : S == 2 ? g_ring2 : g_ring3;
}
__device__ __forceinline__ bf16_t* ring_rt(int s) {
  return s == 0 ? g_ring0 : s == 1 ? g_ring1 : s == 2 ? g_ring2 : g_ring3;
}

// LDS element offset of (row, col) in a row-major tile of width W (bf16) with
// 16-byte chunks XOR-swizzled by the low 4 row bits.
template <int W>
__device__ __forceinline__ int sw(int row, int col) {
  return row * W + ((((col >> 3) ^ (row & 15))) << 3) + (col & 7);
}

// One global_load_lds_dwordx4: every lane copies 16 bytes from gptr into LDS
// at lds_base + 16 * lane. Issued through inline assembly so that the only
// waits on it are the explicit s_waitcnt of the pipeline.
__device__ __forceinline__ void dma16(const void* gptr, const bf16_t* lds_base) {
  // lds_base is the same for the whole wave; make that explicit for the SGPR
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)lds_base)));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m0), "v"(gptr)
               : "memory", "m0");
}

// s_waitcnt vmcnt(N) leaving the other counters unconstrained (gfx9 encoding).
template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// B: block size (the K extent); NC: output columns per workgroup (B, or 256
// at B = 512); TT: tokens per tile. GRAM (B = 128, NC = 128, TT = 64, no
// transpose): the workgroup also accumulates the gram
//   part[split][blk][:, slab NC ..] = X[t, blk]^T C[t, blk cols slab NC ..]
// over its tokens from the same input tiles (C's NC columns ride in each
// ring slot after the input tile), so the backward's gradient apply and its
// gram read the shared operand X once.
template <int B, int NC, int TT, bool TRANS, bool GRAM = false>
struct BlockApply {
  static constexpr int CB = NC / 128;         // 32-wide column blocks per wave
  static constexpr int KS = B / 16;           // MFMA K steps
  static constexpr int RB = TT / 32;          // 32-token row blocks per tile
  static constexpr int STAGE = TT * B;        // elements of one input tile
  static constexpr int LPW = STAGE * 2 / 1024 / 4;  // 1 KB tile loads per wave
  static constexpr int CPT = TT * NC / 8 / kNT;     // 16-byte output chunks per thread
  static constexpr int LPC = GRAM ? TT * NC * 2 / 1024 / 4 : 0;  // 1 KB C-tile loads per wave
  static constexpr int LPT = LPW + LPC;             // loads per wave per tile
  static_assert(STAGE + (GRAM ? TT * NC : 0) <= kStage && TT % 32 == 0 && NC % 128 == 0 && CPT >= 1,
                "tile shape");
  static_assert(!GRAM || (!TRANS && B == 128 && NC == 128 && TT == 64), "gram variant shape");
  // gram: 2 x 2 waves over the B x NC result, wave tile (B/2) x (NC/2)
  static constexpr int GM = B / 2 / 32, GN = NC / 2 / 32;

  const bf16_t* X;
  bf16_t* Y;
  int64_t d, col0, ocol0;  // first input column of the block, first output column
  bool y_tiled;            // Y in the tiled layout (kernels.h)
  int t_begin, t_end, ntiles;
  int tid, lane, wave, nw;
  bf16x8_t bfr[CB][KS];
  const bf16_t* C;  // gram: first of this slab's C columns
  floatx16 gacc[GRAM ? GM : 1][GRAM ? GN : 1];

  // Issues the LDS-bound loads of token tile `tile` into ring slot `dst`.
  __device__ __forceinline__ void load_tile(int tile, bf16_t* dst) {
    const int t0 = t_begin + tile * TT;
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
      const int Q = wave * LPW + q;            // 1 KB piece of the tile
      const int e = Q * 512 + lane * 8;        // element this lane lands on
      const int row = e / B, pch = (e % B) >> 3;
      const int lch = pch ^ (row & 15);
      const int grow = min(t0 + row, t_end - 1);  // rows past the end read a valid row
      dma16(X + (int64_t)grow * d + col0 + lch * 8, dst + Q * 512);
    }
    if constexpr (GRAM) {
#pragma unroll
      for (int q = 0; q < LPC; ++q) {
        const int Q = wave * LPC + q;
        const int e = Q * 512 + lane * 8;
        const int row = e / NC, pch = (e % NC) >> 3;
        const int lch = pch ^ (row & 15);
        const int grow = min(t0 + row, t_end - 1);
        dma16(C + (int64_t)grow * d + lch * 8, dst + STAGE + Q * 512);
      }
    }
  }

  // gram fragment: 8 consecutive tokens (k) x 32 features (m) of a
  // [token][feature] tile of width W, two transposing reads
  template <int W>
  __device__ __forceinline__ bf16x8_t gfrag(const bf16_t* tl, int m0, int k0, int ln) const {
    const int g = ln >> 4, i = ln & 15;
    const int m = m0 + 16 * (g & 1) + 4 * (i & 3);
    short4_t h[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int kk = k0 + 8 * (g >> 1) + 4 * hh + (i >> 2);
      h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(tl + sw<W>(kk, m)));
    }
    union { short4_t s[2]; bf16x8_t v; } u;
    u.s[0] = h[0];
    u.s[1] = h[1];
    return u.v;
  }

  template <int S>
  __device__ __forceinline__ void tile(int t) {
    bf16_t* st = ring<S>();
    // opaque copy of the lane id: keeps the compiler from hoisting this tile's
    // address arithmetic out of the loop (it would hold registers throughout)
    int ln = lane, td = tid;
    asm volatile("" : "+v"(ln), "+v"(td));
    // tile t is in LDS once at most (tiles issued after it) x LPW loads are pending
    if (t + 2 < ntiles) wait_vm<2 * LPT>();
    else if (t + 1 < ntiles) wait_vm<LPT>();
    else wait_vm<0>();
    // this wave's staging writes of tile t-1 have landed (s_waitcnt lgkmcnt(0))
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));
    __builtin_amdgcn_s_barrier();  // every wave's part of tile t landed; slot of t-1 free
    if (t + 3 < ntiles) load_tile(t + 3, ring<(S + 3) & 3>());

    if constexpr (GRAM) {
      const int valid = t_end - (t_begin + t * TT);
      if (valid < TT) {
        // ragged last tile: rows past the end hold a repeated valid token;
        // zero them in the input tile so they add nothing to the gram (their
        // apply outputs are not stored)
        for (int e = td; e < (TT - valid) * B; e += kNT) st[sw<B>(valid + e / B, e % B)] = 0;
        __syncthreads();
      }
      const int wm = wave & 1, wn = wave >> 1;
      const bf16_t* tc = st + STAGE;
#pragma unroll
      for (int kk = 0; kk < TT / 16; ++kk) {
        bf16x8_t fa[GM], fc[GN];
#pragma unroll
        for (int i = 0; i < GM; ++i) fa[i] = gfrag<B>(st, wm * (B / 2) + 32 * i, 16 * kk, ln);
#pragma unroll
        for (int j = 0; j < GN; ++j) fc[j] = gfrag<NC>(tc, wn * (NC / 2) + 32 * j, 16 * kk, ln);
#pragma unroll
        for (int i = 0; i < GM; ++i)
#pragma unroll
          for (int j = 0; j < GN; ++j)
            gacc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fc[j], gacc[i][j], 0, 0, 0);
      }
    }

    floatx16 acc[RB][CB];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int j = 0; j < CB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[r][j][e] = 0.f;
    bf16x8_t af[2][RB];
    auto rd = [&](int ks, bf16x8_t* a) {
#pragma unroll
      for (int r = 0; r < RB; ++r)
        a[r] = *reinterpret_cast<const bf16x8_t*>(st + sw<B>(32 * r + (ln & 31), 16 * ks + 8 * (ln >> 5)));
    };
    rd(0, af[0]);
    static_assert(KS % CPT == 0, "stores spread evenly over the K steps");
    const int tp0 = t_begin + (t - 1) * TT;  // first token of the staged tile t-1
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) rd(ks + 1, af[(ks + 1) & 1]);
      if (t > 0 && ks % (KS / CPT) == 0) store_chunk(ks / (KS / CPT), tp0, td);
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int j = 0; j < CB; ++j)
          acc[r][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j][ks], af[ks & 1][r], acc[r][j], 0, 0, 0);
    }
    __builtin_amdgcn_s_barrier();  // all waves done reading slot S and the staged tile t-1
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        // acc[r][j] holds Y^T: lane l has token 32 r + l % 32 and, for
        // e = 4 g .. 4 g + 3, the four consecutive columns
        // nw + 32 j + 8 g + 4 (l / 32) + (e % 4): one 8-byte LDS write each
        const int m = 32 * r + (ln & 31);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = nw + 32 * j + 8 * g + 4 * (ln >> 5);
          short4_t v;
          v[0] = (short)f32_to_bf16(acc[r][j][4 * g + 0]);
          v[1] = (short)f32_to_bf16(acc[r][j][4 * g + 1]);
          v[2] = (short)f32_to_bf16(acc[r][j][4 * g + 2]);
          v[3] = (short)f32_to_bf16(acc[r][j][4 * g + 3]);
          *reinterpret_cast<short4_t*>(g_out + sw<NC>(m, n)) = v;
        }
      }
    // no barrier: the next tile's first barrier orders these writes before
    // its reads of g_out
  }

  // output chunk q of the staged tile whose first token is t0
  __device__ __forceinline__ void store_chunk(int q, int t0, int td) {
    const int c = td + q * kNT;
    const int row = c / (NC / 8), ch = c % (NC / 8);
    const uint4 v = *reinterpret_cast<const uint4*>(g_out + sw<NC>(row, ch * 8));
    if (t0 + row < t_end) {
      const int64_t off = y_tiled ? tiled_offset(t0 + row, ocol0 + ch * 8, d)
                                  : (int64_t)(t0 + row) * d + ocol0 + ch * 8;
      *reinterpret_cast<uint4*>(Y + off) = v;
    }
  }
};

// Workgroup (split, blk, slab) for NSLAB = B / NC slabs per block: ids are
// unit = split * nb + blk when NSLAB = 1, else 8 NSLAB g + 8 slab + r for
// unit 8 g + r (the slabs of one unit 8 ids apart, on one XCD).
template <int B, int NC, int TT, bool TRANS, bool GRAM = false>
__global__ void __launch_bounds__(kNT)
blockapply_kernel(const bf16_t* __restrict__ X, const bf16_t* __restrict__ Mb, bf16_t* Y, int tokens,
                  int64_t d, int nb, int nsplit, int tok_per_wg, int y_tiled,
                  const bf16_t* C = nullptr, float* __restrict__ part = nullptr) {
  // (Y and C may be one buffer in the gram variant: every element of C is
  // read by the workgroup that writes Y at the same place, before it does)
  typedef BlockApply<B, NC, TT, TRANS, GRAM> K;
  constexpr int NSLAB = B / NC;
  K k;
  k.tid = threadIdx.x;
  k.lane = k.tid & 63;
  k.wave = k.tid >> 6;
  int unit, slab = 0;
  if (NSLAB == 1) {
    unit = blockIdx.x;
  } else {
    unit = (int)(blockIdx.x / (8 * NSLAB)) * 8 + (int)(blockIdx.x & 7);
    slab = (int)(blockIdx.x >> 3) % NSLAB;
  }
  if (unit >= nb * nsplit) return;  // padding id of the last group (uniform, before any barrier)
  const int blk = unit % nb;
  const int split = unit / nb;
  k.t_begin = split * tok_per_wg;
  k.t_end = min(tokens, k.t_begin + tok_per_wg);
  if (k.t_begin >= k.t_end) return;
  k.X = X;
  k.Y = Y;
  k.y_tiled = y_tiled != 0;
  k.d = d;
  k.col0 = (int64_t)blk * B;
  k.ocol0 = k.col0 + slab * NC;
  k.nw = k.wave * (NC / 4);
  k.ntiles = (k.t_end - k.t_begin + TT - 1) / TT;
  if constexpr (GRAM) {
    k.C = C + k.ocol0;
#pragma unroll
    for (int i = 0; i < K::GM; ++i)
#pragma unroll
      for (int j = 0; j < K::GN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) k.gacc[i][j][e] = 0.f;
  }

  const int nt = k.ntiles;
  if constexpr (TRANS) {
    // B(n, k) = M[n][k]: fragment (j, ks) of lane l is 8 consecutive k
    // (16 ks + 8 (l / 32) ..) of slab row nw + 32 j + l % 32, one 16-byte
    // global load each, issued after the first token tiles so that both are
    // in flight together (no LDS staging pass, no barriers before tile 0)
    k.load_tile(0, ring<0>());
    if (nt > 1) k.load_tile(1, ring<1>());
    if (nt > 2) k.load_tile(2, ring<2>());
    const bf16_t* mrow = Mb + (int64_t)blk * B * B + (int64_t)(slab * NC + k.nw + (k.lane & 31)) * B +
                         8 * (k.lane >> 5);
#pragma unroll
    for (int j = 0; j < K::CB; ++j)
#pragma unroll
      for (int ks = 0; ks < K::KS; ++ks)
        k.bfr[j][ks] = *reinterpret_cast<const bf16x8_t*>(mrow + (int64_t)(32 * j) * B + 16 * ks);
  } else {
    // B(n, k) = M[k][n]: the columns slab NC .. of every row of M_k go to LDS
    // (rows spread over the ring slots, in passes when they do not fit), and
    // each fragment (8 consecutive k of column n) comes back with two
    // transposing reads of 4 k each
    const bf16_t* src0 = Mb + (int64_t)blk * B * B + slab * NC;
    constexpr int ROWS_PER_SLOT = kStage / NC;
    constexpr int PASS_ROWS = 4 * ROWS_PER_SLOT < B ? 4 * ROWS_PER_SLOT : B;
    constexpr int NPASS = B / PASS_ROWS;    // the ring holds PASS_ROWS rows at a time
    static_assert(NPASS * PASS_ROWS == B, "whole passes");
    const int lane = k.lane;
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
      for (int c = k.tid; c < PASS_ROWS * NC / 8; c += kNT) {
        const int row = c / (NC / 8), ch = c % (NC / 8);
        bf16_t* slot = ring_rt(row / ROWS_PER_SLOT);
        *reinterpret_cast<uint4*>(slot + sw<NC>(row % ROWS_PER_SLOT, ch * 8)) =
            *reinterpret_cast<const uint4*>(src0 + (int64_t)(pass * PASS_ROWS + row) * B + ch * 8);
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < K::CB; ++j)
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) {
          if ((16 * ks) / PASS_ROWS != pass) continue;
          const int g = lane >> 4, i = lane & 15;
          const int n = k.nw + 32 * j + 16 * (g & 1) + 4 * (i & 3);
          short4_t h[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int kk = 16 * ks + 8 * (g >> 1) + 4 * hh + (i >> 2) - pass * PASS_ROWS;
            h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_short4*)(ring_rt(kk / ROWS_PER_SLOT) + sw<NC>(kk % ROWS_PER_SLOT, n)));
          }
          union { short4_t s[2]; bf16x8_t v; } u;
          u.s[0] = h[0];
          u.s[1] = h[1];
          k.bfr[j][ks] = u.v;
        }
      __syncthreads();  // the ring is restaged, then reused for token tiles
    }
    k.load_tile(0, ring<0>());
    if (nt > 1) k.load_tile(1, ring<1>());
    if (nt > 2) k.load_tile(2, ring<2>());
  }
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
  __syncthreads();  // the last tile is staged
#pragma unroll
  for (int q = 0; q < K::CPT; ++q) k.store_chunk(q, k.t_begin + (nt - 1) * TT, k.tid);
  if constexpr (GRAM) {
    // gram accumulators: lane l of fragment (i, j) holds rows
    // 8 (e / 4) + 4 (l / 32) + e % 4 of the 32-row block and column l % 32
    float* out = part + ((int64_t)split * nb + blk) * B * B + slab * NC;
    const int wm = k.wave & 1, wn = k.wave >> 1, lane = k.lane;
#pragma unroll
    for (int i = 0; i < K::GM; ++i)
#pragma unroll
      for (int j = 0; j < K::GN; ++j) {
        const int n = wn * (NC / 2) + 32 * j + (lane & 31);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = wm * (B / 2) + 32 * i + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
          out[(int64_t)m * B + n] = k.gacc[i][j][e];
        }
      }
  }
}

// Token range of one workgroup: one round of at most 256 workgroups (one per
// CU), token ranges in whole tiles of TT.
int tokens_per_workgroup(int64_t tokens, int64_t d, int B, int NC, int TT) {
  const int nb = (int)(d / B);
  int splits = 256 / (nb * (B / NC));
  const int max_splits = (int)((tokens + TT - 1) / TT);
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int per = (int)((tokens + splits - 1) / splits);
  return (per + TT - 1) / TT * TT;
}

template <int B, int NC, int TT, bool TRANS>
hipError_t launch_b(const bf16_t* X, const bf16_t* M, bf16_t* Y, int64_t tokens, int64_t d,
                    bool y_tiled, hipStream_t s) {
  constexpr int NSLAB = B / NC;
  const int nb = (int)(d / B);
  const int per = tokens_per_workgroup(tokens, d, B, NC, TT);
  const int splits = (int)((tokens + per - 1) / per);
  const int units = nb * splits;
  const int grid = NSLAB == 1 ? units : (units + 7) / 8 * (8 * NSLAB);
  hipLaunchKernelGGL((blockapply_kernel<B, NC, TT, TRANS>), dim3(grid), dim3(kNT), 0, s, X, M, Y,
                     (int)tokens, d, nb, splits, per, (int)y_tiled);
  return hipGetLastError();
}

// One thread per 16-byte chunk of the super blocks: the chunk at (row r,
// columns c0 .. c0 + 7) of super block sb lies in block column c0 / b (b is a
// multiple of 8); it is a row piece of block sb S/b + r / b when that is the
// block's own column, else zeros.
__global__ void __launch_bounds__(kNT)
superblock_kernel(const bf16_t* __restrict__ blocks, int b, int S, int64_t nchunks,
                  bf16_t* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * kNT + threadIdx.x;
  if (c >= nchunks) return;
  const int per_row = S / 8;
  const int64_t row_all = c / per_row;           // row over all super blocks
  const int sb = (int)(row_all / S), r = (int)(row_all % S);
  const int c0 = (int)(c % per_row) * 8;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (r / b == c0 / b) {
    const int64_t blk = (int64_t)sb * (S / b) + r / b;
    v = *reinterpret_cast<const uint4*>(blocks + (blk * b + r % b) * b + c0 % b);
  }
  *reinterpret_cast<uint4*>(out + c * 8) = v;
}

}  // namespace

int superblock_size(DType t, int64_t d, int b) {
  return (t == DType::BF16 && (b == 32 || b == 64) && d % 128 == 0) ? 128 : 0;
}

hipError_t launch_superblocks(const void* blocks, int64_t nblocks, int b, int S, void* out,
                              hipStream_t s) {
  if (b % 8 != 0 || S % b != 0 || nblocks % (S / b) != 0) return hipErrorInvalidValue;
  const int64_t nchunks = nblocks / (S / b) * S * S / 8;
  const int64_t grid = (nchunks + kNT - 1) / kNT;
  hipLaunchKernelGGL(superblock_kernel, dim3((unsigned)grid), dim3(kNT), 0, s,
                     static_cast<const bf16_t*>(blocks), b, S, nchunks, static_cast<bf16_t*>(out));
  return hipGetLastError();
}

bool blockgramapply_supported(DType t, int64_t d, int b) {
  return t == DType::BF16 && (b == 128 || b == 256) && d % b == 0;
}

template <int B, int NC, int TT>
hipError_t launch_gram_b(const void* X, const void* M, const void* C, void* Y, float* part,
                         int64_t tokens, int64_t d, int max_split, int* nsplit, bool y_tiled,
                         hipStream_t s) {
  constexpr int NSLAB = B / NC;
  const int nb = (int)(d / B);
  // one round of at most 256 workgroups, whole tiles per split, and no more
  // splits than the caller's partial buffer holds
  int splits = 256 / (nb * NSLAB);
  const int max_tiles = (int)((tokens + TT - 1) / TT);
  if (splits > max_tiles) splits = max_tiles;
  if (splits > max_split) splits = max_split;
  if (splits < 1) splits = 1;
  int per = (int)((tokens + splits - 1) / splits);
  per = (per + TT - 1) / TT * TT;
  splits = (int)((tokens + per - 1) / per);  // every split holds at least one token
  const int units = nb * splits;
  const int grid = NSLAB == 1 ? units : (units + 7) / 8 * (8 * NSLAB);
  hipLaunchKernelGGL((blockapply_kernel<B, NC, TT, false, true>), dim3(grid), dim3(kNT), 0, s,
                     static_cast<const bf16_t*>(X), static_cast<const bf16_t*>(M),
                     static_cast<bf16_t*>(Y), (int)tokens, d, nb, splits, per, (int)y_tiled,
                     static_cast<const bf16_t*>(C), part);
  *nsplit = splits;
  return hipGetLastError();
}

hipError_t launch_blockgramapply(const void* X, const void* M, const void* C, void* Y, float* part,
                                 int64_t tokens, int64_t d, int b, int max_split, int* nsplit,
                                 bool y_tiled, hipStream_t s) {
  if ((b != 128 && b != 256) || d % b != 0 || tokens < 1 || max_split < 1) return hipErrorInvalidValue;
  if (y_tiled && (tokens % kTileRows != 0 || C == Y)) return hipErrorInvalidValue;
  if (b == 256)
    return launch_gramapply256(X, M, C, Y, part, tokens, d, max_split, nsplit, y_tiled, s);
  return launch_gram_b<128, 128, 64>(X, M, C, Y, part, tokens, d, max_split, nsplit, y_tiled, s);
}

bool blockapply_supported(DType t, int64_t d, int b) {
  return t == DType::BF16 && (b == 128 || b == 256 || b == 512) && d % b == 0;
}

int64_t blockapply_tokens_per_workgroup(int64_t tokens, int64_t d, int b) {
  if (b == 512) return tokens_per_workgroup(tokens, d, 512, 256, 32);
  if (b == 256) return tokens_per_workgroup(tokens, d, 256, 256, 64);
  return tokens_per_workgroup(tokens, d, 128, 128, 64);
}

hipError_t launch_blockapply(const void* X, const void* M, void* Y, int64_t tokens, int64_t d, int b,
                             bool transpose, bool y_tiled, hipStream_t s) {
  if (y_tiled && tokens % kTileRows != 0) return hipErrorInvalidValue;
  const bf16_t* x = static_cast<const bf16_t*>(X);
  const bf16_t* m = static_cast<const bf16_t*>(M);
  bf16_t* y = static_cast<bf16_t*>(Y);
  const bool yt = y_tiled;
  if (b == 512) return transpose ? launch_b<512, 256, 32, true>(x, m, y, tokens, d, yt, s)
                                 : launch_b<512, 256, 32, false>(x, m, y, tokens, d, yt, s);
  if (b == 256) return transpose ? launch_b<256, 256, 64, true>(x, m, y, tokens, d, yt, s)
                                 : launch_b<256, 256, 64, false>(x, m, y, tokens, d, yt, s);
  return transpose ? launch_b<128, 128, 64, true>(x, m, y, tokens, d, yt, s)
                   : launch_b<128, 128, 64, false>(x, m, y, tokens, d, yt, s);
}

}  // namespace poetx
