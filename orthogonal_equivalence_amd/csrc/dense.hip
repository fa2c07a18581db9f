// The dense W0 products of the POET-X layer on bf16 MFMA: the forward
// Z = U W0^T (W0 is [d_out][d_in], so both operands are K-contiguous) and the
// backward g_U = g_Z W0 (W0 read along its rows, i.e. N-contiguous). W0 is
// the frozen weight of the layer (gist.science technical summary of "POET-X:
// Memory-efficient LLM Training by Scaling Orthogonal Transformation",
// section 2 Methodik); these two products carry almost all of the layer's
// arithmetic.
//
// C[M][N] = A[M][K] B(n, k) with B(n, k) = B[n][k] (K-major) or B[k][n]
// (N-major); bf16 in and out, float32 accumulation.
//
// One workgroup of four waves, one per SIMD, computes a 256 x 256 tile; each
// wave owns a 128 x 128 quarter as 8 x 8 tiles of v_mfma_f32_16x16x32_bf16
// whose 256 accumulator registers live in AGPRs. A 128 x 128 wave tile is
// the largest the register file allows and reads the fewest operand bytes
// from LDS per product (64 KB per 32-deep K tile for the workgroup, against
// 96 KB for eight 128 x 64 waves). Measured on gfx950 at one wave per SIMD:
// a back-to-back 16x16x32 stream issues every 16.2 cycles, and every
// ds_read_b128 interleaved with it costs about 8 more, so operand bytes read
// into registers, not the products, set the pace; the fewer of them, the
// less power the LDS draws, and the chip's clock under this load is power
// limited.
//
// K tiles of 32 are copied from global memory straight into a 4-slot LDS
// ring with global_load_lds_dwordx4 (no register staging, no LDS store
// instructions), three tiles ahead of the products. Every wave issues its
// share of the copies, one 1 KB piece after each row of eight products, so
// the address unit sees a steady stream rather than a burst that would block
// the issuing wave (in-order issue: a blocked copy holds back the products
// behind it). Per K tile: the first row of products runs on registers, then
// one barrier publishes the next K tile and frees the slot of the current
// one, then the other seven rows run while the next tile's fragments are
// read, two per row, into the second register set.
//
// The products are inline asm with the accumulator tied to an AGPR operand:
// with the compiler's builtin the register allocator rotated the
// accumulators between AGPRs on every iteration (hundreds of
// v_accvgpr_mov per K tile). The first K tile uses a zero addend, so the
// accumulators are never cleared by VALU writes. The compiler does not see
// the asm products, so the wait states before the epilogue reads them are
// explicit.
//
// LDS layouts (16-byte chunks XOR-swizzled so that the fragment reads are
// free of bank conflicts):
//   K-major tile  [256 rows][32 k]  (64-byte rows): chunk c of row r at
//                 c ^ ((r >> 1) & 3). Measured on gfx950 (whose LDS returns
//                 256 bytes per clock for these reads): this pattern of
//                 ds_read_b128 fragment reads streams 234 B/clk per CU, while
//                 c ^ (((r >> 1) & 3) ^ ((r >> 3) & 1)), r & 3, (r >> 2) & 3
//                 or no swizzle all give 128 B/clk (two-way conflicts);
//   N-major tile  [32 k][256 n]     (512-byte rows): chunk c of row k at
//                 c ^ 2 (k & 3), read with the transposing ds_read_b64_tr_b16;
//   epilogue      [256 m][256 n] bf16 (the whole ring): chunk c of row m at
//                 c ^ (m & 15).
// The products are issued as D' = B A^T (the operand roles swapped), so each
// lane ends up holding four consecutive output columns of one row and stages
// them with one 8-byte LDS write; the staged tile leaves as 16-byte stores of
// whole 512-byte row segments.
//
// A may also be in the tiled layout (kernels.h): each 256 x 32 piece of the
// matrix one contiguous 16 KB block, so a K tile of a 256-row panel is one
// block and every copy reads 1 KB of consecutive bytes (eight whole 128-byte
// lines), where the row-major layout gives each copy 16 half lines of 64
// bytes; on the 8B MLP-up shapes the forward took 7 % less time and the
// backward 4 % less. A K-major B may be tiled the same way (the forward's
// weight, where a caller widens INT8 codes into a buffer of its own).
//
// M and N must be at least 256 and K a multiple of 32: a tile that would
// cross the end of M or N is shifted back to end there (it recomputes, and
// rewrites with identical values, part of its neighbour), so no load or
// store needs a bounds test. The kernel is persistent: workgroup g computes
// tiles g, g + G, ... (G = grid size, a multiple of 8, so each workgroup
// stays on one XCD's share of the grouped tile order).
#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace poetx {
namespace {

constexpr int BM = 256, BN = 256, BK = 32;
constexpr int NW = 4, NT = 64 * NW;        // one wave per SIMD
constexpr int FM = 8, FN = 8;              // 16-row / 16-column fragments per wave
constexpr int TILE = BM * BK;              // bf16 elements of one operand tile (16 KB)
constexpr int SLOT = 2 * TILE;             // A and B tiles
constexpr int NSLOT = 4;
constexpr int RING = NSLOT * SLOT;         // 128 KB, also the epilogue's staging tile
constexpr int PPW = TILE * 2 / 1024 / NW;  // 1 KB pieces per wave per operand tile
constexpr int LPW = 2 * PPW;               // copies per wave per K tile
static_assert(RING == BM * BN, "the epilogue stages the whole output tile in the ring");
static_assert(PPW == 4 && LPW == 8, "one copy after each of the eight rows of products");

// 1 KB alignment: the fragment addressing XORs bits 4..6 of element offsets
__shared__ __attribute__((aligned(1024))) bf16_t g_dense_lds[RING];

__device__ __forceinline__ int kmaj_swz(int row) { return (row >> 1) & 3; }
__device__ __forceinline__ int nmaj_swz(int k) { return (k & 3) << 1; }
__device__ __forceinline__ int nmaj_off(int k, int n) {
  return k * BN + ((((n >> 3) ^ nmaj_swz(k))) << 3) + (n & 7);
}
__device__ __forceinline__ int stage_off(int m, int n) {
  return m * BN + ((((n >> 3) ^ (m & 15))) << 3) + (n & 7);
}

// One global_load_lds_dwordx4 in the scalar-base form: lane l copies the 16
// bytes at sbase + voff into LDS at m0 + 16 l.
__device__ __forceinline__ void dma16_sb(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(m0), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

__device__ __forceinline__ const bf16_t* uniform_ptr(const bf16_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const bf16_t*>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <bool B_KMAJ>
struct Dense {
  const bf16_t* baseA;  // wave-uniform bases of the current tile's A and B panels
  const bf16_t* baseB;
  int64_t stepA, stepB; // elements between consecutive K tiles of A and of B
  bool a_tiled;         // A in the tiled layout (then M % 256 == 0 and lda == K)
                        // (a tiled K-major B likewise: N % 256 == 0, ldb == K)
  uint32_t offA, offB;  // per-lane byte offsets of this wave's first piece at k = 0
  uint32_t strA, strB;  // bytes between this wave's consecutive pieces
  uint32_t lds0;        // LDS byte address of the ring, wave-uniform
  int wave, lane, wm, wn;
  int rdA, rdB;         // per-lane element offsets of fragment 0 within a tile
  floatx4 acc[FM][FN];
  bf16x8_t fa[2][FM], fb[2][FN];

  __device__ __forceinline__ void init(int64_t lda, int64_t ldb, bool tiled, bool b_tiled) {
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    lane = threadIdx.x & 63;
    wm = wave & 1;
    wn = wave >> 1;
    lds0 = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)g_dense_lds)));
    a_tiled = tiled;
    stepA = tiled ? (int64_t)BM * BK : BK;
    stepB = B_KMAJ ? (b_tiled ? (int64_t)BN * BK : BK) : (int64_t)BK * ldb;
    const int r = lane & 15;
    rdA = (wm * 128 + r) * BK + (((lane >> 4) ^ kmaj_swz(r)) << 3);
    if (B_KMAJ) {
      rdB = (wn * 128 + r) * BK + (((lane >> 4) ^ kmaj_swz(r)) << 3);
    } else {
      // fragment j adds 16 j columns: chunk index + 2 j, which the swizzle
      // turns into an XOR of the element offset with 16 j
      const int k = 8 * (lane >> 4) + (r >> 2);
      rdB = nmaj_off(k, wn * 128 + 4 * (r & 3));
    }
    // wave w copies pieces q = w + 4 j (j < 4) of each operand tile: K-major
    // piece q holds rows 16 q .. 16 q + 15, N-major piece q holds k rows
    // 2 q, 2 q + 1; either way the swizzle of a lane's data is the same for
    // all of its pieces
    const int row = 16 * wave + (lane >> 2);
    const int c = (lane & 3) ^ kmaj_swz(row);
    // (tiled: the rows of a K tile are 32 elements apart within its block)
    const int64_t rsa = tiled ? BK : lda;
    offA = (uint32_t)(row * rsa + 8 * c) * 2u;
    strA = (uint32_t)(16 * NW * rsa) * 2u;
    if (B_KMAJ) {
      const int64_t rsb = b_tiled ? BK : ldb;
      offB = (uint32_t)(row * rsb + 8 * c) * 2u;
      strB = (uint32_t)(16 * NW * rsb) * 2u;
    } else {
      const int k = 2 * wave + (lane >> 5);
      const int cn = (lane & 31) ^ nmaj_swz(k);
      offB = (uint32_t)(k * ldb + 8 * cn) * 2u;
      strB = (uint32_t)(2 * NW * ldb) * 2u;
    }
  }

  // panels of the output tile at (m0, n0) (wholly inside M x N)
  __device__ __forceinline__ void set_tile(const bf16_t* A, const bf16_t* B, int64_t lda,
                                           int64_t ldb, int m0, int n0) {
    // (tiled: the panel's blocks start at row m0 of the row-major count,
    // since a panel of 256 rows holds 256 lda elements)
    baseA = uniform_ptr(A + (int64_t)m0 * lda);
    baseB = uniform_ptr(B_KMAJ ? B + (int64_t)n0 * ldb : B + n0);
  }

  // piece J of K tile t of operand OP (0: A, 1: B) into ring slot S
  template <int S, int OP, int J>
  __device__ __forceinline__ void dma(int t) {
    const uint32_t m = lds0 + (uint32_t)(S * SLOT * 2 + OP * TILE * 2 + (wave + NW * J) * 1024);
    if (OP == 0)
      dma16_sb(uniform_ptr(baseA + (int64_t)t * stepA), offA + J * strA, m);
    else
      dma16_sb(uniform_ptr(baseB + (int64_t)t * stepB), offB + J * strB, m);
  }
  template <int S>
  __device__ __forceinline__ void issue(int t) {
    dma<S, 0, 0>(t); dma<S, 0, 1>(t); dma<S, 0, 2>(t); dma<S, 0, 3>(t);
    dma<S, 1, 0>(t); dma<S, 1, 1>(t); dma<S, 1, 2>(t); dma<S, 1, 3>(t);
  }

  // A fragment I (rows 16 I .. of this wave's 128; lane l holds row l % 16,
  // k = 8 (l / 16) .. +7) from ring slot S into set P
  template <int S, int P, int I>
  __device__ __forceinline__ void read_a() {
    fa[P][I] = *reinterpret_cast<const bf16x8_t*>(g_dense_lds + S * SLOT + rdA + 512 * I);
  }
  // B fragment J (16 of this wave's columns) likewise
  template <int S, int P, int J>
  __device__ __forceinline__ void read_b() {
    const bf16_t* sb = g_dense_lds + S * SLOT + TILE;
    if (B_KMAJ) {
      fb[P][J] = *reinterpret_cast<const bf16x8_t*>(sb + rdB + 512 * J);
    } else {
      const int o = rdB ^ (16 * J);
      union { short4_t h[2]; bf16x8_t v; } u;
      u.h[0] = ds_read_tr4(sb + o);
      u.h[1] = ds_read_tr4(sb + o + 4 * BN);
      fb[P][J] = u.v;
    }
  }

  // acc[I][J] += B fragment J x A fragment I (D' = B A^T: lane l holds
  // output row 16 I + l % 16, columns 16 J + 4 (l / 16) .. +3)
  template <int P, int I, int J, bool FIRST>
  __device__ __forceinline__ void mma() {
    if (FIRST)
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0"
                   : "=a"(acc[I][J])
                   : "v"(fb[P][J]), "v"(fa[P][I]));
    else
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                   : "+a"(acc[I][J])
                   : "v"(fb[P][J]), "v"(fa[P][I]));
  }
  template <int P, int I, bool FIRST>
  __device__ __forceinline__ void mma_row() {
    mma<P, I, 0, FIRST>(); mma<P, I, 1, FIRST>(); mma<P, I, 2, FIRST>(); mma<P, I, 3, FIRST>();
    mma<P, I, 4, FIRST>(); mma<P, I, 5, FIRST>(); mma<P, I, 6, FIRST>(); mma<P, I, 7, FIRST>();
  }

  // K tile t, held in ring slot S, its fragments in set P. STEADY: tiles
  // t+1 .. t+4 all exist, so every step below is taken. FIRST: t == 0.
  template <int S, int P, bool STEADY, bool FIRST = false>
  __device__ __forceinline__ void tile(int t, int ntiles) {
    constexpr int S1 = (S + 1) & 3;
    const bool more = STEADY || t + 1 < ntiles;
    const bool iss = STEADY || t + 4 < ntiles;
    mma_row<P, 0, FIRST>();
    __builtin_amdgcn_sched_barrier(0);
    if (more) {
      // this wave's part of tile t+1 landed (tiles t+2, t+3 may still be in
      // flight) and its reads of tile t are done; after the barrier every
      // part has landed and slot S is free
      if (STEADY || t + 3 < ntiles) wait_vm<2 * LPW>();
      else if (t + 2 < ntiles) wait_vm<LPW>();
      else wait_vm<0>();
      wait_lds();
      barrier_nofence();
    }
    if (iss) dma<S, 0, 0>(t + 4);
    __builtin_amdgcn_sched_barrier(0);
#define POETX_DENSE_ROW(I)                                                          \
  mma_row<P, I, FIRST>();                                                           \
  if (iss) dma<S, (I) / 4, (I) % 4>(t + 4);                                         \
  if (more) { read_a<S1, P ^ 1, (I) - 1>(); read_b<S1, P ^ 1, (I) - 1>(); }         \
  __builtin_amdgcn_sched_barrier(0);
    POETX_DENSE_ROW(1) POETX_DENSE_ROW(2) POETX_DENSE_ROW(3) POETX_DENSE_ROW(4)
    POETX_DENSE_ROW(5) POETX_DENSE_ROW(6) POETX_DENSE_ROW(7)
#undef POETX_DENSE_ROW
    if (more) { read_a<S1, P ^ 1, 7>(); read_b<S1, P ^ 1, 7>(); }
  }

  // copies of the first (up to) four K tiles of the current output tile
  __device__ __forceinline__ void prefetch(int ntiles) {
    issue<0>(0);
    if (ntiles > 1) issue<1>(1);
    if (ntiles > 2) issue<2>(2);
    if (ntiles > 3) issue<3>(3);
  }

  // every part of K tile 0 landed (this wave's earlier stores too: the
  // count is conservative); its fragments read
  __device__ __forceinline__ void start(int ntiles) {
    if (ntiles > 3) wait_vm<3 * LPW>();
    else if (ntiles > 2) wait_vm<2 * LPW>();
    else if (ntiles > 1) wait_vm<LPW>();
    else wait_vm<0>();
    barrier_nofence();
    read_a<0, 0, 0>(); read_a<0, 0, 1>(); read_a<0, 0, 2>(); read_a<0, 0, 3>();
    read_a<0, 0, 4>(); read_a<0, 0, 5>(); read_a<0, 0, 6>(); read_a<0, 0, 7>();
    read_b<0, 0, 0>(); read_b<0, 0, 1>(); read_b<0, 0, 2>(); read_b<0, 0, 3>();
    read_b<0, 0, 4>(); read_b<0, 0, 5>(); read_b<0, 0, 6>(); read_b<0, 0, 7>();
  }

  __device__ __forceinline__ void mainloop(int ntiles) {
    // tile 0 writes the accumulators; then slots 1, 2, 3, 0, 1, ...
    if (ntiles > 4) tile<0, 0, true, true>(0, ntiles);
    else tile<0, 0, false, true>(0, ntiles);
    int t = 1;
    for (; t + 8 <= ntiles; t += 4) {  // branch-free steady state
      tile<1, 1, true>(t, ntiles);
      tile<2, 0, true>(t + 1, ntiles);
      tile<3, 1, true>(t + 2, ntiles);
      tile<0, 0, true>(t + 3, ntiles);
    }
    // the last 0 .. 7 tiles
    if (t < ntiles) tile<1, 1, false>(t++, ntiles);
    if (t < ntiles) tile<2, 0, false>(t++, ntiles);
    if (t < ntiles) tile<3, 1, false>(t++, ntiles);
    if (t < ntiles) tile<0, 0, false>(t++, ntiles);
    if (t < ntiles) tile<1, 1, false>(t++, ntiles);
    if (t < ntiles) tile<2, 0, false>(t++, ntiles);
    if (t < ntiles) tile<3, 1, false>(t++, ntiles);
    // wait states between the last products and the VALU reads of their
    // results in the epilogue (more than any 16x16x32 product needs)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }

  // accumulators -> bf16 staging tile (the whole ring) -> 16-byte stores of
  // whole 512-byte row segments; the ring is free again on return
  __device__ __forceinline__ void epilogue(bf16_t* __restrict__ C, int64_t ldc, int m0, int n0) {
    // opaque copies of the lane and thread ids: keeps the compiler from
    // hoisting the epilogue's address arithmetic out of the tile loop
    int ln = lane, tid = (int)threadIdx.x;
    asm volatile("" : "+v"(ln), "+v"(tid));
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int m = wm * 128 + 16 * i + (ln & 15);
        const int n = wn * 128 + 16 * j + 4 * (ln >> 4);
        union { bf16_t h[4]; uint2 v; } u;
#pragma unroll
        for (int e = 0; e < 4; ++e) u.h[e] = f32_to_bf16(acc[i][j][e]);
        *reinterpret_cast<uint2*>(g_dense_lds + stage_off(m, n)) = u.v;
        __builtin_amdgcn_sched_barrier(0);  // one fragment's registers at a time
      }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < BM * BN / 8 / NT; ++q) {
      const int c = tid + q * NT;
      const int rl = c >> 5, nl = (c & 31) * 8;
      const uint4 v = *reinterpret_cast<const uint4*>(g_dense_lds + stage_off(rl, nl));
      *reinterpret_cast<uint4*>(C + (int64_t)(m0 + rl) * ldc + n0 + nl) = v;
    }
    wait_lds();
    barrier_nofence();
  }

  // ---- forward with the R-apply fused (B K-major, 256 x 256 R blocks) ----
  // Y tile = Z tile R_k^T for the output tile's R block R_k (its 256 columns
  // are one block): the bf16 Z tile staged in the ring is the A operand, R_k's
  // rows are the B fragments (loaded from global memory, the block stays in
  // L2), K = 256 in 8 steps of 32, accumulated in the same AGPRs. Without
  // KEEP_Z only Y leaves the CU (a run-time test there made the compiler
  // spill ~0.5 KB per lane).
  template <int S>
  __device__ __forceinline__ void load_r(const bf16_t* rrow) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[S & 1][j] = *reinterpret_cast<const bf16x8_t*>(rrow + j * 16 * 256 + S * 32);
  }
  template <int S>
  __device__ __forceinline__ void r_step(const bf16_t* rrow, int ln) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[S & 1][i] = *reinterpret_cast<const bf16x8_t*>(
          g_dense_lds + stage_off(wm * 128 + 16 * i + (ln & 15), 32 * S + 8 * (ln >> 4)));
    if (S + 1 < 8) load_r<(S + 1) & 7>(rrow);
    mma_row<S & 1, 0, S == 0>(); mma_row<S & 1, 1, S == 0>();
    mma_row<S & 1, 2, S == 0>(); mma_row<S & 1, 3, S == 0>();
    mma_row<S & 1, 4, S == 0>(); mma_row<S & 1, 5, S == 0>();
    mma_row<S & 1, 6, S == 0>(); mma_row<S & 1, 7, S == 0>();
    __builtin_amdgcn_sched_barrier(0);
  }
  // the accumulators -> bf16 -> staging tile (the whole ring)
  __device__ __forceinline__ void stage_acc(int ln) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int m = wm * 128 + 16 * i + (ln & 15);
        const int n = wn * 128 + 16 * j + 4 * (ln >> 4);
        union { bf16_t h[4]; uint2 v; } u;
#pragma unroll
        for (int e = 0; e < 4; ++e) u.h[e] = f32_to_bf16(acc[i][j][e]);
        *reinterpret_cast<uint2*>(g_dense_lds + stage_off(m, n)) = u.v;
        __builtin_amdgcn_sched_barrier(0);
      }
  }
  // the staging tile -> 16-byte stores of whole row segments of C (row stride ldc)
  __device__ __forceinline__ void store_staged(bf16_t* __restrict__ C, int64_t ldc, int m0, int n0,
                                               int tid) {
#pragma unroll
    for (int q = 0; q < BM * BN / 8 / NT; ++q) {
      const int c = tid + q * NT;
      const int rl = c >> 5, nl = (c & 31) * 8;
      const uint4 v = *reinterpret_cast<const uint4*>(g_dense_lds + stage_off(rl, nl));
      *reinterpret_cast<uint4*>(C + (int64_t)(m0 + rl) * ldc + n0 + nl) = v;
    }
  }
  template <bool KEEP_Z>
  __device__ __forceinline__ void epilogue_fused(bf16_t* __restrict__ C, int64_t ldc, int m0,
                                                 int n0, const bf16_t* __restrict__ Rk,
                                                 bf16_t* __restrict__ Y, int64_t ldy) {
    int ln = lane, tid = (int)threadIdx.x;
    asm volatile("" : "+v"(ln), "+v"(tid));
    // B fragment (j, step s) of lane l: R_k row wn 128 + 16 j + l % 16,
    // columns 32 s + 8 (l / 16) .. + 7
    const bf16_t* rrow = Rk + (wn * 128 + (ln & 15)) * 256 + 8 * (ln >> 4);
    load_r<0>(rrow);  // in flight while Z is staged
    stage_acc(ln);
    wait_lds();
    barrier_nofence();  // (no memory fence: nothing waits for the loads or stores here)
    r_step<0>(rrow, ln); r_step<1>(rrow, ln); r_step<2>(rrow, ln); r_step<3>(rrow, ln);
    r_step<4>(rrow, ln); r_step<5>(rrow, ln); r_step<6>(rrow, ln); r_step<7>(rrow, ln);
    // wait states before the VALU reads of the products' results
    asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (KEEP_Z) store_staged(C, ldc, m0, n0, tid);  // Z
    wait_lds();
    barrier_nofence();  // every wave is done reading the staged Z
    stage_acc(ln);
    wait_lds();
    barrier_nofence();  // Z's stores stay in flight
    store_staged(Y, ldy, m0, n0, tid);  // Y
    wait_lds();
    barrier_nofence();
  }
};

// nbatch independent products of the same shape, product q at A + q sA,
// B + q sB, C + q sC (the block-diagonal products of b >= 512 blocks run as
// one batched launch); their output tiles form one grid of num_mt x
// (nbatch num_nt) tiles, products side by side along N.
template <bool B_KMAJ, bool FUSE_R = false, bool KEEP_Z = true>
__global__ void __launch_bounds__(NT)
dense_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, bf16_t* __restrict__ C,
             int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc,
             const bf16_t* __restrict__ R, bf16_t* __restrict__ Y, int64_t ldy, int nbatch,
             int64_t sA, int64_t sB, int64_t sC, int a_tiled, int b_tiled) {
  const int num_mt = (M + BM - 1) / BM, num_nt = (N + BN - 1) / BN;
  const int total = num_mt * num_nt * nbatch;
  const int ntiles = K / BK;
  int tile = blockIdx.x;
  if (tile >= total) return;

  Dense<B_KMAJ> d;
  d.init(lda, ldb, a_tiled != 0, B_KMAJ && b_tiled != 0);
  for (;;) {
    int mt, ntb;
    xcd_grouped_tile_at(tile, total, num_mt, num_nt * nbatch, mt, ntb);
    const int q = ntb / num_nt, nt = ntb - q * num_nt;
    const int m0 = min(mt * BM, M - BM), n0 = min(nt * BN, N - BN);
    d.set_tile(A + q * sA, B + q * sB, lda, ldb, m0, n0);
    d.prefetch(ntiles);
    d.start(ntiles);
    d.mainloop(ntiles);
    wait_lds();
    barrier_nofence();  // every wave is done with the ring
    if constexpr (FUSE_R)
      d.template epilogue_fused<KEEP_Z>(C, ldc, m0, n0, R + (int64_t)(n0 / 256) * 256 * 256, Y,
                                        ldy);
    else
      d.epilogue(C + q * sC, ldc, m0, n0);
    tile += (int)gridDim.x;
    if (tile >= total) break;
  }
}

}  // namespace

bool dense_supported(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc) {
  // the per-lane copy offsets within one 256-row (or 32-row) panel are 32-bit
  return M >= BM && N >= BN && K >= BK && K % BK == 0 && N % 8 == 0 && lda % 8 == 0 &&
         ldb % 8 == 0 && ldc % 8 == 0 && M <= INT32_MAX && N <= INT32_MAX && K <= INT32_MAX &&
         lda <= (1 << 22) && ldb <= (1 << 22);
}

namespace {
hipError_t dense_grid(int64_t M, int64_t N, int* grid_out) {
  const int tiles = (int)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
  // one workgroup per CU (the register and LDS footprints allow no more),
  // rounded down to a multiple of the 8 XCDs
  static thread_local int cached_dev = -1, cached_cus = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev != cached_dev) {
    e = hipDeviceGetAttribute(&cached_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cached_dev = dev;
  }
  int grid = cached_cus >= 8 ? cached_cus & ~7 : cached_cus;
  if (grid > tiles) grid = tiles;
  if (grid < 1) grid = 1;
  *grid_out = grid;
  return hipSuccess;
}
}  // namespace

hipError_t launch_dense(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                        int64_t lda, int64_t ldb, int64_t ldc, bool b_kmajor, bool a_tiled,
                        bool b_tiled, hipStream_t s) {
  if (a_tiled && (M % BM != 0 || lda != K)) return hipErrorInvalidValue;
  if (b_tiled && (!b_kmajor || N % BN != 0 || ldb != K)) return hipErrorInvalidValue;
  int grid = 0;
  hipError_t e = dense_grid(M, N, &grid);
  if (e != hipSuccess) return e;
  const bf16_t* a = static_cast<const bf16_t*>(A);
  const bf16_t* b = static_cast<const bf16_t*>(B);
  bf16_t* c = static_cast<bf16_t*>(C);
  if (b_kmajor)
    hipLaunchKernelGGL((dense_kernel<true, false>), dim3(grid), dim3(NT), 0, s, a, b, c, (int)M,
                       (int)N, (int)K, lda, ldb, ldc, nullptr, nullptr, (int64_t)0, 1, (int64_t)0,
                       (int64_t)0, (int64_t)0, (int)a_tiled, (int)b_tiled);
  else
    hipLaunchKernelGGL((dense_kernel<false, false>), dim3(grid), dim3(NT), 0, s, a, b, c, (int)M,
                       (int)N, (int)K, lda, ldb, ldc, nullptr, nullptr, (int64_t)0, 1, (int64_t)0,
                       (int64_t)0, (int64_t)0, (int)a_tiled, (int)b_tiled);
  return hipGetLastError();
}

hipError_t launch_dense_batched(const void* A, const void* B, void* C, int64_t M, int64_t N,
                                int64_t K, int64_t lda, int64_t ldb, int64_t ldc, bool b_kmajor,
                                int64_t nbatch, int64_t sA, int64_t sB, int64_t sC,
                                hipStream_t s) {
  if (nbatch < 1 || nbatch * ((N + BN - 1) / BN) * ((M + BM - 1) / BM) > INT32_MAX)
    return hipErrorInvalidValue;
  int grid = 0;
  hipError_t e = dense_grid(M, N * nbatch, &grid);
  if (e != hipSuccess) return e;
  const bf16_t* a = static_cast<const bf16_t*>(A);
  const bf16_t* b = static_cast<const bf16_t*>(B);
  bf16_t* c = static_cast<bf16_t*>(C);
  if (b_kmajor)
    hipLaunchKernelGGL((dense_kernel<true, false>), dim3(grid), dim3(NT), 0, s, a, b, c, (int)M,
                       (int)N, (int)K, lda, ldb, ldc, nullptr, nullptr, (int64_t)0, (int)nbatch,
                       sA, sB, sC, 0, 0);
  else
    hipLaunchKernelGGL((dense_kernel<false, false>), dim3(grid), dim3(NT), 0, s, a, b, c, (int)M,
                       (int)N, (int)K, lda, ldb, ldc, nullptr, nullptr, (int64_t)0, (int)nbatch,
                       sA, sB, sC, 0, 0);
  return hipGetLastError();
}

bool dense_fused_r_supported(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                             int64_t ldc, int64_t ldy) {
  return dense_supported(M, N, K, lda, ldb, ldc) && N % 256 == 0 && ldy % 8 == 0;
}

hipError_t launch_dense_fused_r(const void* A, const void* B, void* C, int64_t M, int64_t N,
                                int64_t K, int64_t lda, int64_t ldb, int64_t ldc, const void* R,
                                void* Y, int64_t ldy, bool a_tiled, bool b_tiled, hipStream_t s) {
  if (a_tiled && (M % BM != 0 || lda != K)) return hipErrorInvalidValue;
  if (b_tiled && (N % BN != 0 || ldb != K)) return hipErrorInvalidValue;
  int grid = 0;
  hipError_t e = dense_grid(M, N, &grid);
  if (e != hipSuccess) return e;
  if (C)
    hipLaunchKernelGGL((dense_kernel<true, true>), dim3(grid), dim3(NT), 0, s,
                       static_cast<const bf16_t*>(A), static_cast<const bf16_t*>(B),
                       static_cast<bf16_t*>(C), (int)M, (int)N, (int)K, lda, ldb, ldc,
                       static_cast<const bf16_t*>(R), static_cast<bf16_t*>(Y), ldy, 1, (int64_t)0,
                       (int64_t)0, (int64_t)0, (int)a_tiled, (int)b_tiled);
  else
    hipLaunchKernelGGL((dense_kernel<true, true, false>), dim3(grid), dim3(NT), 0, s,
                       static_cast<const bf16_t*>(A), static_cast<const bf16_t*>(B), nullptr,
                       (int)M, (int)N, (int)K, lda, ldb, ldc, static_cast<const bf16_t*>(R),
                       static_cast<bf16_t*>(Y), ldy, 1, (int64_t)0, (int64_t)0, (int64_t)0,
                       (int)a_tiled, (int)b_tiled);
  return hipGetLastError();
}

}  // namespace poetx
