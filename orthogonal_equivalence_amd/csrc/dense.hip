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
// One workgroup (8 waves, 2 x 4, each 128 x 64 as 8 x 4 tiles of
// v_mfma_f32_16x16x32_bf16, two waves per SIMD) computes a 256 x 256 tile;
// waves 0-3 issue the operand loads and waves 4-7 write the output, so each
// wave's vmcnt only counts its own kind of access. On random operands the
// 16x16x32 shape sustains a markedly higher rate than 32x32x16 under the
// chip's power limit, so it is the one used here. K tiles of 32 are copied
// from global memory straight into a 4-slot LDS ring with
// global_load_lds_dwordx4 (no register staging, no LDS store instructions),
// three tiles ahead of the MFMAs. Each K tile is one MFMA step; the barrier
// that publishes the next tile sits between the two halves of the current
// tile's MFMAs, and the next tile's fragments are read into a second register
// set while the second half runs.
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
//                 c ^ 2 (k & 3), read with the transposing ds_read_b64_tr_b16.
// M and N must be at least 256 and K a multiple of 32: a tile that would
// cross the end of M or N is shifted back to end there (it recomputes, and
// rewrites with identical values, part of its neighbour), so no load or
// store needs a bounds test.
#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace poetx {
namespace {

constexpr int BM = 256, BN = 256, BK = 32;
constexpr int NWAVE = 8;                  // 2 x (NWAVE / 2) waves
constexpr int NT = 64 * NWAVE;
constexpr int TN = 2 * BN / NWAVE;        // wave tile: 128 rows x TN columns
constexpr int FN = TN / 16;               // 16-column B fragments per wave
constexpr int TILE = BM * BK;             // bf16 elements of one operand tile
constexpr int SLOT = 2 * TILE;            // A and B tiles
constexpr int NSLOT = 4;
constexpr int NLOADW = NWAVE / 2;         // waves 0 .. NLOADW-1 issue the loads
constexpr int PPW = 16 / NLOADW;          // 1 KB pieces per loading wave per operand tile
constexpr int LPW = 2 * PPW;              // 1 KB loads per loading wave per K tile
constexpr int SROWS = 64;                 // output rows staged per epilogue pass
constexpr int RING = NSLOT * SLOT;
constexpr int LDS_ELEMS = RING + SROWS * BN;  // 160 KB: ring + epilogue staging

// 1 KB alignment: the fragment addressing XORs bits 4..6 of element offsets
__shared__ __attribute__((aligned(1024))) bf16_t g_dense_lds[LDS_ELEMS];

// element offset of (row, col) in the epilogue staging tile [SROWS][BN]:
// 16-byte chunks XOR-swizzled by bits 2..3 of the row
__device__ __forceinline__ int stage_off(int row, int col) {
  return RING + row * BN + ((((col >> 3) ^ (((row >> 2) & 3) << 1))) << 3) + (col & 7);
}

// swizzle of a K-major row: depends only on row % 16, so the fragments of
// one wave (16-row steps) share one address pattern
__device__ __forceinline__ int kmaj_swz(int row) { return (row >> 1) & 3; }
__device__ __forceinline__ int kmaj_off(int row, int chunk) {
  return row * BK + ((chunk ^ kmaj_swz(row)) << 3);
}
__device__ __forceinline__ int nmaj_swz(int k) { return (k & 3) << 1; }
__device__ __forceinline__ int nmaj_off(int k, int n) {
  return k * BN + ((((n >> 3) ^ nmaj_swz(k))) << 3) + (n & 7);
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
  // wave-uniform bases of the current tile's A and B panels; per-lane byte
  // offsets of this (loading) wave's first 1 KB load per operand at k = 0
  // (its other loads add a wave-uniform stride to the base)
  const bf16_t* baseA;
  const bf16_t* baseB;
  int64_t stepB;   // elements between consecutive K tiles of B
  int64_t pieceA, pieceB;  // elements between this wave's consecutive loads
  uint32_t offA, offB;
  uint32_t lds0;  // LDS byte address of the ring, wave-uniform
  int wave, lane, wm, wn;
  bool loader;    // this wave issues the tile loads
  int rdA, rdB;   // per-lane element offsets of fragment 0 within a tile
  floatx4 acc[8][FN];
  bf16x8_t fa[8], fb[2][FN];

  __device__ __forceinline__ void init(int64_t ldb) {
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    lane = threadIdx.x & 63;
    wm = wave & 1;
    wn = wave >> 1;
    loader = wave < NLOADW;
    lds0 = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)g_dense_lds)));
    stepB = B_KMAJ ? BK : (int64_t)BK * ldb;
    const int r = lane & 15;
    rdA = (wm * 128 + r) * BK + (((lane >> 4) ^ kmaj_swz(r)) << 3);
    if (B_KMAJ) {
      rdB = (wn * TN + r) * BK + (((lane >> 4) ^ kmaj_swz(r)) << 3);
    } else {
      // fragment j adds 16 j columns: chunk index + 2 j, which the swizzle
      // turns into an XOR of the element offset with 16 j
      const int k = 8 * (lane >> 4) + (r >> 2);
      rdB = nmaj_off(k, wn * TN + 4 * (r & 3));
    }
  }

  // load addressing of the output tile at (m0, n0) (wholly inside M x N).
  // Loading wave w issues pieces q = w + NLOADW j (j < PPW) of each operand
  // tile: K-major piece q holds rows 16 q .. 16 q + 15, N-major piece q
  // holds k rows 2 q, 2 q + 1; either way the swizzle of a lane's data is
  // the same for all of its pieces.
  __device__ __forceinline__ void set_tile(const bf16_t* A, const bf16_t* B, int64_t lda,
                                           int64_t ldb, int m0, int n0) {
    baseA = uniform_ptr(A + (int64_t)m0 * lda);
    baseB = uniform_ptr(B_KMAJ ? B + (int64_t)n0 * ldb : B + n0);
    const int w = wave % NLOADW;
    const int row = 16 * w + (lane >> 2);
    const int c = (lane & 3) ^ kmaj_swz(row);
    offA = (uint32_t)(row * lda + 8 * c) * 2u;
    pieceA = 16 * NLOADW * lda;
    if (B_KMAJ) {
      offB = (uint32_t)(row * ldb + 8 * c) * 2u;
      pieceB = 16 * NLOADW * ldb;
    } else {
      const int k = 2 * w + (lane >> 5);
      const int cn = (lane & 31) ^ nmaj_swz(k);
      offB = (uint32_t)(k * ldb + 8 * cn) * 2u;
      pieceB = 2 * NLOADW * ldb;
    }
  }

  // loads of K tile t into ring slot S (loading waves only)
  template <int S>
  __device__ __forceinline__ void issue(int t) {
    const uint32_t m = lds0 + (uint32_t)(S * SLOT * 2 + wave * 1024);
#pragma unroll
    for (int j = 0; j < PPW; ++j)
      dma16_sb(uniform_ptr(baseA + (int64_t)t * BK + j * pieceA), offA, m + NLOADW * 1024 * j);
#pragma unroll
    for (int j = 0; j < PPW; ++j)
      dma16_sb(uniform_ptr(baseB + (int64_t)t * stepB + j * pieceB), offB,
               m + TILE * 2 + NLOADW * 1024 * j);
  }

  // A fragment i: rows 16 i .. of this wave's 128, lane l holds row l % 16,
  // k = 8 (l / 16) .. +7; B fragments likewise over this wave's columns.
  // A fragments i0 .. i1-1 (rows 16 i .. of this wave's 128; lane l holds
  // row l % 16, k = 8 (l / 16) .. +7) from ring slot S
  template <int S, int I0, int I1>
  __device__ __forceinline__ void read_a() {
    const bf16_t* s = g_dense_lds + S * SLOT;
#pragma unroll
    for (int i = I0; i < I1; ++i) fa[i] = *reinterpret_cast<const bf16x8_t*>(s + rdA + 512 * i);
  }
  // B fragments j0 .. j1-1 (16 of this wave's columns each) from ring slot S
  // into set P
  template <int S, int P, int J0 = 0, int J1 = FN>
  __device__ __forceinline__ void read_b() {
    const bf16_t* sb = g_dense_lds + S * SLOT + TILE;
    if (B_KMAJ) {
#pragma unroll
      for (int j = J0; j < J1; ++j) fb[P][j] = *reinterpret_cast<const bf16x8_t*>(sb + rdB + 512 * j);
    } else {
      // recomputed per read (one XOR) rather than held in registers
      int rb = rdB;
      asm volatile("" : "+v"(rb));
#pragma unroll
      for (int j = J0; j < J1; ++j) {
        const int o = rb ^ (16 * j);
        union { short4_t h[2]; bf16x8_t v; } u;
        u.h[0] = ds_read_tr4(sb + o);
        u.h[1] = ds_read_tr4(sb + o + 4 * BN);
        fb[P][j] = u.v;
      }
    }
  }

  template <int I0, int P, int J0 = 0, int J1 = FN>
  __device__ __forceinline__ void mma_rows() {
#pragma unroll
    for (int i = I0; i < I0 + 4; ++i)
#pragma unroll
      for (int j = J0; j < J1; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[P][j], acc[i][j], 0, 0, 0);
  }

  // K tile t, held in ring slot S, its B fragments in set P. The fragments
  // of tile t+1 are read as those of tile t are consumed, which keeps the
  // live fragment registers near one set: after the barrier that publishes
  // tile t+1, A rows 0..3 and the first half of B; after the MFMAs on the
  // second half of B, the rest of B; after the last MFMAs, A rows 4..7.
  // STEADY: tiles t+1 .. t+4 all exist, so every step below is taken
  template <int S, int P, bool STEADY>
  __device__ __forceinline__ void tile(int t, int ntiles) {
    mma_rows<0, P>();
    __builtin_amdgcn_sched_barrier(0);  // keep these MFMAs ahead of the waits
    const bool more = STEADY || t + 1 < ntiles;
    if (more) {
      // tile t+1 landed (each loading wave's part; tiles t+2 and t+3 may
      // still be in flight); then every part, and every wave is done with
      // slot S
      if (loader) {
        if (STEADY || t + 3 < ntiles) wait_vm<2 * LPW>();
        else if (t + 2 < ntiles) wait_vm<LPW>();
        else wait_vm<0>();
      }
      wait_lds();
      barrier_nofence();
      if (loader && (STEADY || t + 4 < ntiles)) issue<S>(t + 4);
      read_a<(S + 1) & 3, 0, 4>();
      read_b<(S + 1) & 3, P ^ 1, 0, FN / 2>();
    }
    mma_rows<4, P, FN / 2, FN>();
    __builtin_amdgcn_sched_barrier(0);
    if (more) read_b<(S + 1) & 3, P ^ 1, FN / 2, FN>();
    mma_rows<4, P, 0, FN / 2>();
    __builtin_amdgcn_sched_barrier(0);
    if (more) read_a<(S + 1) & 3, 4, 8>();
  }

  // loads of the first (up to) four K tiles of the current output tile
  __device__ __forceinline__ void prefetch(int ntiles) {
    if (!loader) return;
    issue<0>(0);
    if (ntiles > 1) issue<1>(1);
    if (ntiles > 2) issue<2>(2);
    if (ntiles > 3) issue<3>(3);
  }

  // every part of K tile 0 landed; its fragments read
  __device__ __forceinline__ void start(int ntiles) {
    if (loader) {
      if (ntiles > 3) wait_vm<3 * LPW>();
      else if (ntiles > 2) wait_vm<2 * LPW>();
      else if (ntiles > 1) wait_vm<LPW>();
      else wait_vm<0>();
    }
    barrier_nofence();
    read_a<0, 0, 8>();
    read_b<0, 0>();
  }

  __device__ __forceinline__ void mainloop(int ntiles) {
    int t = 0;
    for (; t + 8 <= ntiles; t += 4) {  // branch-free steady state
      tile<0, 0, true>(t, ntiles);
      tile<1, 1, true>(t + 1, ntiles);
      tile<2, 0, true>(t + 2, ntiles);
      tile<3, 1, true>(t + 3, ntiles);
    }
    // the last 1 .. 7 tiles
    if (t < ntiles) tile<0, 0, false>(t++, ntiles);
    if (t < ntiles) tile<1, 1, false>(t++, ntiles);
    if (t < ntiles) tile<2, 0, false>(t++, ntiles);
    if (t < ntiles) tile<3, 1, false>(t++, ntiles);
    if (t < ntiles) tile<0, 0, false>(t++, ntiles);
    if (t < ntiles) tile<1, 1, false>(t++, ntiles);
    if (t < ntiles) tile<2, 0, false>(t++, ntiles);
  }

  // accumulators -> bf16 -> 16-byte row segments of C, SROWS rows per pass
  // through the staging tile; the waves that do not load write to global
  // memory, so the loading waves' counters only ever see their own loads
  __device__ __forceinline__ void epilogue(bf16_t* __restrict__ C, int64_t ldc, int m0, int n0) {
    // opaque copies of the lane and thread ids: keeps the compiler from
    // hoisting the epilogue's address arithmetic out of the tile loop, where
    // it would hold registers through the main loop
    int ln = lane, tid = (int)threadIdx.x - 64 * NLOADW;
    asm volatile("" : "+v"(ln), "+v"(tid));
#pragma unroll
    for (int pass = 0; pass < BM / SROWS; ++pass) {
      if (wm == (pass >> 1)) {
        const int i0 = 4 * (pass & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int n = wn * TN + 16 * j + (ln & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 16 * i + 4 * (ln >> 4) + e;
              g_dense_lds[stage_off(r, n)] = f32_to_bf16(acc[i0 + i][j][e]);
            }
          }
      }
      __syncthreads();
      if (!loader) {
#pragma unroll
        for (int q = 0; q < SROWS * BN / 8 / (NT - 64 * NLOADW); ++q) {
          const int c = tid + q * (NT - 64 * NLOADW);
          const int rl = c >> 5, nl = (c & 31) * 8;
          const int m = m0 + pass * SROWS + rl, n = n0 + nl;
          const uint4 v = *reinterpret_cast<const uint4*>(g_dense_lds + stage_off(rl, nl));
          *reinterpret_cast<uint4*>(C + (int64_t)m * ldc + n) = v;
        }
      }
      __syncthreads();
    }
  }
};

// Persistent: workgroup g computes output tiles g, g + G, ... (G = grid
// size, a multiple of 8, so each workgroup stays on one XCD's share of the
// grouped tile order). The first K tiles of the next output tile are loaded
// while the current one is written out.
template <bool B_KMAJ>
__global__ void __launch_bounds__(NT)
dense_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, bf16_t* __restrict__ C,
             int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc) {
  const int num_mt = (M + BM - 1) / BM, num_nt = (N + BN - 1) / BN;
  const int total = num_mt * num_nt;
  const int ntiles = K / BK;
  int tile = blockIdx.x;
  if (tile >= total) return;

  Dense<B_KMAJ> d;
  d.init(ldb);
  int mt, nt;
  xcd_grouped_tile_at(tile, total, num_mt, num_nt, mt, nt);
  d.set_tile(A, B, lda, ldb, min(mt * BM, M - BM), min(nt * BN, N - BN));
  d.prefetch(ntiles);
  for (;;) {
    const int m0 = min(mt * BM, M - BM), n0 = min(nt * BN, N - BN);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) d.acc[i][j][e] = 0.f;
    d.start(ntiles);
    d.mainloop(ntiles);
    wait_lds();
    barrier_nofence();  // every wave is done with the ring
    const int next = tile + (int)gridDim.x;
    if (next < total) {
      xcd_grouped_tile_at(next, total, num_mt, num_nt, mt, nt);
      d.set_tile(A, B, lda, ldb, min(mt * BM, M - BM), min(nt * BN, N - BN));
      d.prefetch(ntiles);
    }
    d.epilogue(C, ldc, m0, n0);
    if (next >= total) break;
    tile = next;
  }
}

}  // namespace

bool dense_supported(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc) {
  return M >= BM && N >= BN && K >= BK && K % BK == 0 && N % 8 == 0 && lda % 8 == 0 &&
         ldb % 8 == 0 && ldc % 8 == 0 && M <= INT32_MAX && N <= INT32_MAX && K <= INT32_MAX;
}

hipError_t launch_dense(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                        int64_t lda, int64_t ldb, int64_t ldc, bool b_kmajor, hipStream_t s) {
  const int tiles = (int)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
  // one workgroup per CU (the LDS footprint allows no more), rounded down to
  // a multiple of the 8 XCDs
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
  const bf16_t* a = static_cast<const bf16_t*>(A);
  const bf16_t* b = static_cast<const bf16_t*>(B);
  bf16_t* c = static_cast<bf16_t*>(C);
  if (b_kmajor)
    hipLaunchKernelGGL(dense_kernel<true>, dim3(grid), dim3(NT), 0, s, a, b, c, (int)M, (int)N,
                       (int)K, lda, ldb, ldc);
  else
    hipLaunchKernelGGL(dense_kernel<false>, dim3(grid), dim3(NT), 0, s, a, b, c, (int)M, (int)N,
                       (int)K, lda, ldb, ldc);
  return hipGetLastError();
}

}  // namespace poetx
