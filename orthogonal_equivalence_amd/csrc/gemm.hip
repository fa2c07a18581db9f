// Batched split-K GEMM on CDNA4 matrix cores (MFMA), used for every
// contraction of the POET-X layer: the block-diagonal applies of R and P
// (batched over blocks), the dense W0 products, the token-reduction grams
// G_R and G_P (split over tokens), and the Cayley VJP products.
//
// One workgroup computes a BM x BN tile of one batch (and one K split). Both
// operand tiles are staged in LDS K-contiguous, 128 bytes per row, with the
// 16-byte chunks of row r XOR-swizzled by f(r) = ((r >> 1) ^ ((r & 1) << 2)) & 7
// so that the MFMA fragment reads of 8 or 16 consecutive rows hit distinct
// banks. Two LDS buffers: the next tile's global loads are issued before the
// MFMAs on the current one, and one barrier per K step separates the LDS
// write of the next buffer from the reads of the current one. An operand
// that is contiguous along M/N in global memory (a transposed access, e.g.
// the token-major activations of the grams, or W0 in the backward) is loaded
// as VEC x VEC sub-blocks of 16-byte rows and transposed in registers on the
// way to LDS.
//
// Workgroups are dispatched round-robin over the 8 XCDs; the tile order is
// remapped so each XCD works on a contiguous range of a grouped (GROUP_M
// row tiles at a time) ordering, which keeps the A and B panels that
// concurrently running tiles share in that XCD's L2.
//
// Configurations: bf16 256x256x64 tiles, 2x2 waves of 128x128 with
// v_mfma_f32_32x32x16_bf16 (large shapes); bf16 128x128x64 with
// v_mfma_f32_16x16x32_bf16 (small shapes); float32 64x64x32 with
// v_mfma_f32_16x16x4_f32. Accumulation is float32 throughout.
#include "common.h"
#include "kernels.h"

namespace poetx {
namespace {

__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ ((row & 1) << 2)) & 7; }

// (batch, tile) of this workgroup for a grid of (tiles, batch, splits).
// Workgroups are dispatched to the 8 XCDs round-robin by linear index, so
// the linear index is remapped to give each XCD a contiguous run of the
// batch-major tile order: all tiles of a batch entry (a b x b block) then
// run on one XCD and share its L2, instead of every XCD streaming every
// block's operands. Inside a batch entry, tiles go in groups of 8 tile rows.
__device__ __forceinline__ void batched_tile(int num_mt, int num_nt, int& bt, int& mt, int& nt) {
  const int T = num_mt * num_nt;  // == gridDim.x
  const int nwg = (int)(gridDim.x * gridDim.y);
  int w = (int)(blockIdx.x + gridDim.x * blockIdx.y);
  if ((nwg & 7) == 0) w = (w & 7) * (nwg >> 3) + (w >> 3);
  bt = w / T;
  const int t = w - bt * T;
  constexpr int GROUP_M = 8;
  const int per_group = GROUP_M * num_nt;
  const int group = t / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(num_mt - first_m, GROUP_M);
  const int in_group = t - group * per_group;
  mt = first_m + in_group % gsize;
  nt = in_group / gsize;
}

// Transpose of a VEC x VEC block held as VEC 16-byte rows: out[c] holds
// element c of every input row, in row order.
template <typename T> struct Transpose;
template <> struct Transpose<bf16_t> {  // 8 x 8 bf16
  __device__ static uint4 column(const uint4* v, int c) {
    // dword d of the output holds rows 2d (low half) and 2d+1 (high half)
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    auto pick = [&](int r) -> uint32_t {
      const uint4& q = v[r];
      const int d = c >> 1;
      return d == 0 ? q.x : d == 1 ? q.y : d == 2 ? q.z : q.w;
    };
    uint4 o;
    o.x = __builtin_amdgcn_perm(pick(1), pick(0), sel);
    o.y = __builtin_amdgcn_perm(pick(3), pick(2), sel);
    o.z = __builtin_amdgcn_perm(pick(5), pick(4), sel);
    o.w = __builtin_amdgcn_perm(pick(7), pick(6), sel);
    return o;
  }
};
template <> struct Transpose<float> {  // 4 x 4 float
  __device__ static uint4 column(const uint4* v, int c) {
    auto pick = [&](int r) -> uint32_t {
      const uint4& q = v[r];
      return c == 0 ? q.x : c == 1 ? q.y : c == 2 ? q.z : q.w;
    };
    return make_uint4(pick(0), pick(1), pick(2), pick(3));
  }
};

// LDS tile: ROWS rows of BK elements (128 bytes), swizzled chunks.
template <typename TIn, int BK>
struct LdsLayout {
  static constexpr int VEC = ElemTraits<TIn>::kVec;
  static_assert(BK * sizeof(TIn) == 128, "LDS rows are 128 bytes");
  __device__ static int chunk_off(int row, int chunk) { return row * BK + ((chunk ^ swz(row)) * VEC); }
  __device__ static int elem_off(int row, int k) { return chunk_off(row, k / VEC) + (k % VEC); }
};

// Global -> register -> LDS staging of one operand tile. Only whole 16-byte
// vectors are moved: the host guarantees that K extents of K-major operands
// and row extents of MN-major operands are multiples of VEC, so a vector is
// either entirely inside the operand or entirely outside (then zero).
template <typename TIn, int ROWS, int BK, int NT, bool KMAJ>
struct TileLoader {
  static constexpr int VEC = ElemTraits<TIn>::kVec;
  typedef LdsLayout<TIn, BK> L;
  // K-major: one 16-byte chunk (VEC consecutive k of one row) per item.
  // MN-major: one VEC(k) x VEC(row) sub-block per item.
  static constexpr int ITEMS = KMAJ ? ROWS * BK / VEC : (ROWS / VEC) * (BK / VEC);
  static constexpr int PER_THREAD = (ITEMS + NT - 1) / NT;
  static constexpr int REGS = KMAJ ? PER_THREAD : PER_THREAD * VEC;
  static constexpr bool EXACT = (ITEMS % NT) == 0;

  uint4 r[REGS];

  // MN-major items run k-chunk fastest across lanes: the 8 lanes that store
  // one row's 8 chunks then cover all banks (conflict-free transposed stores),
  // and each global load instruction still reads whole 128-byte lines.
  __device__ static void item_pos(int item, int& a, int& b) {
    if (KMAJ) { a = item / (BK / VEC); b = item % (BK / VEC); }  // row, chunk
    else { a = item / (BK / VEC); b = item % (BK / VEC); }       // row block, k block
  }

  // base points at element (row 0, k 0) of this batch; rows/k are global
  // indices. Rows >= rext or k >= kend read as zero. Tiles that lie wholly
  // inside the operand take a path without per-vector bounds tests.
  __device__ __forceinline__ void load(const TIn* __restrict__ base, int64_t ld, int r0, int rext,
                                       int k0, int kend, int tid) {
    const bool full = (r0 + ROWS <= rext) && (k0 + BK <= kend);
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int item = tid + i * NT;
      int ia, ib;
      item_pos(item, ia, ib);
      const bool live = EXACT || item < ITEMS;
      if (KMAJ) {
        const int gr = r0 + ia, gk = k0 + ib * VEC;
        const TIn* src = base + (int64_t)gr * ld + gk;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (full) {
          if (live) v = *reinterpret_cast<const uint4*>(src);
        } else if (live && gr < rext && gk < kend) {
          v = *reinterpret_cast<const uint4*>(src);
        }
        r[i] = v;
      } else {
        const int gr = r0 + ia * VEC;
        const bool rows_ok = live && gr < rext;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const int gk = k0 + ib * VEC + e;
          const TIn* src = base + (int64_t)gk * ld + gr;
          uint4 v = make_uint4(0, 0, 0, 0);
          if (full) {
            if (live) v = *reinterpret_cast<const uint4*>(src);
          } else if (rows_ok && gk < kend) {
            v = *reinterpret_cast<const uint4*>(src);
          }
          r[i * VEC + e] = v;
        }
      }
    }
  }

  __device__ __forceinline__ void store(TIn* __restrict__ s, int tid) const {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int item = tid + i * NT;
      if (!EXACT && item >= ITEMS) continue;
      int ia, ib;
      item_pos(item, ia, ib);
      if (KMAJ) {
        *reinterpret_cast<uint4*>(s + L::chunk_off(ia, ib)) = r[i];
      } else {
#pragma unroll
        for (int c = 0; c < VEC; ++c)
          *reinterpret_cast<uint4*>(s + L::chunk_off(ia * VEC + c, ib)) =
              Transpose<TIn>::column(&r[i * VEC], c);
      }
    }
  }
};

// MFMA shapes. `load` reads the fragment of rows [row0, row0 + M) at K
// offset kk; `out_row` maps accumulator element e of a lane to its row in
// the M x M output tile (the column is lane % M).
template <typename TIn, int MI> struct Mfma;

template <> struct Mfma<bf16_t, 32> {
  static constexpr int M = 32, KSTEP = 16, NACC = 16;
  typedef bf16x8_t Frag;
  typedef floatx16 Acc;
  template <int BK>
  __device__ static Frag load(const bf16_t* s, int row0, int kk, int lane) {
    const int row = row0 + (lane & 31);
    return *reinterpret_cast<const bf16x8_t*>(s + LdsLayout<bf16_t, BK>::chunk_off(row, (kk >> 3) + (lane >> 5)));
  }
  __device__ static Acc mma(Frag a, Frag b, Acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static int out_row(int e, int lane) { return (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3); }
};

template <> struct Mfma<bf16_t, 16> {
  static constexpr int M = 16, KSTEP = 32, NACC = 4;
  typedef bf16x8_t Frag;
  typedef floatx4 Acc;
  template <int BK>
  __device__ static Frag load(const bf16_t* s, int row0, int kk, int lane) {
    const int row = row0 + (lane & 15);
    return *reinterpret_cast<const bf16x8_t*>(s + LdsLayout<bf16_t, BK>::chunk_off(row, (kk >> 3) + (lane >> 4)));
  }
  __device__ static Acc mma(Frag a, Frag b, Acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static int out_row(int e, int lane) { return 4 * (lane >> 4) + e; }
};

template <> struct Mfma<float, 16> {
  static constexpr int M = 16, KSTEP = 4, NACC = 4;
  typedef float Frag;
  typedef floatx4 Acc;
  template <int BK>
  __device__ static Frag load(const float* s, int row0, int kk, int lane) {
    return s[LdsLayout<float, BK>::elem_off(row0 + (lane & 15), kk + (lane >> 4))];
  }
  __device__ static Acc mma(Frag a, Frag b, Acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static int out_row(int e, int lane) { return 4 * (lane >> 4) + e; }
};

template <typename TIn, typename TOut, bool A_KMAJ, bool B_KMAJ, int BM, int BN, int BK, int WM,
          int WN, int MI>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_kernel(const GemmParams p) {
  typedef Mfma<TIn, MI> Op;
  constexpr int NT = 64 * WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / MI, FN = TN / MI;
  constexpr int STAGE = (BM + BN) * BK;
  static_assert(TM % MI == 0 && TN % MI == 0, "wave tile must be a multiple of the MFMA tile");
  static_assert(BK % Op::KSTEP == 0, "bad K tile");

  // The output tile is staged through LDS (rows padded by 16 bytes) and
  // written with 16-byte stores; float32 outputs of the 256 x 256 tile do not
  // fit and are stored directly from the accumulators.
  constexpr int CPAD = 16 / sizeof(TOut);
  constexpr int CLD = BN + CPAD;
  constexpr size_t RING_BYTES = sizeof(TIn) * 2 * STAGE;
  constexpr size_t C_BYTES = sizeof(TOut) * BM * CLD;
  constexpr bool LDS_EPI = C_BYTES <= 144 * 1024;
  constexpr size_t SMEM_BYTES = (LDS_EPI && C_BYTES > RING_BYTES) ? C_BYTES : RING_BYTES;
  __shared__ __attribute__((aligned(16))) char smem_raw[SMEM_BYTES];
  TIn* smem = reinterpret_cast<TIn*>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;

  const int num_mt = (p.M + BM - 1) / BM;
  const int num_nt = (p.N + BN - 1) / BN;
  int bt, mt, nt;
  batched_tile(num_mt, num_nt, bt, mt, nt);
  const bool last = (bt == p.batch - 1);
  const int Mx = last ? p.M_last : p.M;
  const int Nx = last ? p.N_last : p.N;
  const int Kx = last ? p.K_last : p.K;
  const int m0 = mt * BM;
  const int n0 = nt * BN;
  if (m0 >= Mx || n0 >= Nx) return;  // whole workgroup: tile outside a ragged last batch

  const int kbeg = blockIdx.z * p.kchunk;
  const int kend = min(Kx, kbeg + p.kchunk);
  const int ntiles = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

  const bool seg2 = bt >= p.batch_split;
  const int sb = seg2 ? bt - p.batch_split : bt;  // batch index within its segment
  const TIn* A = static_cast<const TIn*>(seg2 ? p.A2 : p.A) + (int64_t)sb * p.sA;
  const TIn* B = static_cast<const TIn*>(seg2 ? p.B2 : p.B) + (int64_t)sb * p.sB;

  TileLoader<TIn, BM, BK, NT, A_KMAJ> la;
  TileLoader<TIn, BN, BK, NT, B_KMAJ> lb;

  typename Op::Acc acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < Op::NACC; ++e) acc[i][j][e] = 0.0f;

  // Software pipeline over K tiles: while the MFMAs consume tile t from one
  // LDS buffer, the registers holding tile t+1 are written to the other
  // buffer (free since the previous barrier) and the global loads of tile
  // t+2 are issued into the same registers. One barrier per tile.
  constexpr int NK = BK / Op::KSTEP;
  static_assert(NK >= 2, "the pipeline needs at least two MFMA steps per K tile");
  if (ntiles > 0) {
    la.load(A, p.lda, m0, Mx, kbeg, kend, tid);
    lb.load(B, p.ldb, n0, Nx, kbeg, kend, tid);
    la.store(smem, tid);
    lb.store(smem + BM * BK, tid);
    if (ntiles > 1) {
      la.load(A, p.lda, m0, Mx, kbeg + BK, kend, tid);
      lb.load(B, p.ldb, n0, Nx, kbeg + BK, kend, tid);
    }
    __syncthreads();
  }

  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    const TIn* As = smem + cur * STAGE;
    const TIn* Bs = As + BM * BK;
    TIn* nxt = smem + (cur ^ 1) * STAGE;
    typename Op::Frag af[2][FM], bfr[2][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) af[0][i] = Op::template load<BK>(As, wm * TM + i * MI, 0, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) bfr[0][j] = Op::template load<BK>(Bs, wn * TN + j * MI, 0, lane);
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      const int fb = s & 1;
      if (s + 1 < NK) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[fb ^ 1][i] = Op::template load<BK>(As, wm * TM + i * MI, (s + 1) * Op::KSTEP, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bfr[fb ^ 1][j] = Op::template load<BK>(Bs, wn * TN + j * MI, (s + 1) * Op::KSTEP, lane);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = Op::mma(af[fb][i], bfr[fb][j], acc[i][j]);
      if (s == 0 && t + 1 < ntiles) {
        la.store(nxt, tid);
        lb.store(nxt + BM * BK, tid);
      }
      if (s == 1 && t + 2 < ntiles) {
        const int k0 = kbeg + (t + 2) * BK;
        la.load(A, p.lda, m0, Mx, k0, kend, tid);
        lb.load(B, p.ldb, n0, Nx, k0, kend, tid);
      }
    }
    __syncthreads();
  }

  TOut* C = static_cast<TOut*>(seg2 ? p.C2 : p.C) + (int64_t)sb * p.sC +
            (int64_t)blockIdx.z * p.sC_split;
  const void* Dv = seg2 ? p.D2 : p.D;
  const TOut* D = Dv ? static_cast<const TOut*>(Dv) + (int64_t)sb * p.sD : nullptr;
  if constexpr (LDS_EPI) {
    // accumulators -> LDS tile (row-major, padded) -> 16-byte row segments,
    // with alpha and beta * D applied on the way out
    TOut* cs = reinterpret_cast<TOut*>(smem_raw);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = wn * TN + j * MI + (lane % MI);
#pragma unroll
        for (int e = 0; e < Op::NACC; ++e) {
          const int m = wm * TM + i * MI + Op::out_row(e, lane);
          cs[m * CLD + n] = ElemTraits<TOut>::from_f32(acc[i][j][e]);
        }
      }
    __syncthreads();
    constexpr int V = ElemTraits<TOut>::kVec;
    constexpr int CHUNKS = BM * BN / V;
    const bool vec_ok = (Nx - n0 >= BN) || ((Nx % V) == 0);
#pragma unroll 1
    for (int c = tid; c < CHUNKS; c += NT) {
      const int ml = c / (BN / V), nl = (c % (BN / V)) * V;
      const int m = m0 + ml, n = n0 + nl;
      if (m >= Mx || n >= Nx) continue;
      union { uint4 u; TOut e[V]; } v;
      v.u = *reinterpret_cast<const uint4*>(cs + ml * CLD + nl);
      const bool whole = vec_ok && n + V <= Nx;
      if (p.alpha != 1.0f || D) {
#pragma unroll
        for (int t = 0; t < V; ++t) {
          float f = p.alpha * ElemTraits<TOut>::to_f32(v.e[t]);
          if (D && n + t < Nx) {
            const int64_t di = p.d_trans ? (int64_t)(n + t) * p.ldd + m : (int64_t)m * p.ldd + n + t;
            f += p.beta * ElemTraits<TOut>::to_f32(D[di]);
          }
          v.e[t] = ElemTraits<TOut>::from_f32(f);
        }
      }
      TOut* dst = C + (int64_t)m * p.ldc + n;
      if (whole) {
        *reinterpret_cast<uint4*>(dst) = v.u;
      } else {
#pragma unroll
        for (int t = 0; t < V; ++t)
          if (n + t < Nx) dst[t] = v.e[t];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn * TN + j * MI + (lane % MI);
#pragma unroll
        for (int e = 0; e < Op::NACC; ++e) {
          const int m = m0 + wm * TM + i * MI + Op::out_row(e, lane);
          if (m < Mx && n < Nx) {
            float v = p.alpha * acc[i][j][e];
            if (D) {
              const int64_t di = p.d_trans ? (int64_t)n * p.ldd + m : (int64_t)m * p.ldd + n;
              v += p.beta * ElemTraits<TOut>::to_f32(D[di]);
            }
            store_as<TOut>(C + (int64_t)m * p.ldc + n, v);
          }
        }
      }
    }
  }
}

struct Big { static constexpr int BM = 256, BN = 256, BK = 64, WM = 2, WN = 2, MI = 32; };
struct SmallBf16 { static constexpr int BM = 128, BN = 128, BK = 64, WM = 2, WN = 2, MI = 16; };
struct TinyBf16 { static constexpr int BM = 64, BN = 64, BK = 64, WM = 2, WN = 2, MI = 16; };
struct SmallF32 { static constexpr int BM = 64, BN = 64, BK = 32, WM = 2, WN = 2, MI = 16; };
// float32 products with M >= 128: each wave 64 x 32, eight MFMAs per six
// fragment reads per k step (the 64 x 64 tile does four per four)
struct MidF32 { static constexpr int BM = 128, BN = 64, BK = 32, WM = 2, WN = 2, MI = 16; };

template <typename TIn, typename TOut, bool AK, bool BK_, typename C>
hipError_t launch_cfg(const GemmParams& p, hipStream_t stream) {
  const int num_mt = (p.M + C::BM - 1) / C::BM;
  const int num_nt = (p.N + C::BN - 1) / C::BN;
  dim3 grid(num_mt * num_nt, p.batch, p.ksplit);
  dim3 block(64 * C::WM * C::WN);
  hipLaunchKernelGGL((gemm_kernel<TIn, TOut, AK, BK_, C::BM, C::BN, C::BK, C::WM, C::WN, C::MI>),
                     grid, block, 0, stream, p);
  return hipGetLastError();
}

template <typename TIn, typename TOut, typename C>
hipError_t launch_layout(bool ak, bool bk, const GemmParams& p, hipStream_t stream) {
  if (ak && bk) return launch_cfg<TIn, TOut, true, true, C>(p, stream);
  if (ak && !bk) return launch_cfg<TIn, TOut, true, false, C>(p, stream);
  if (!ak && !bk) return launch_cfg<TIn, TOut, false, false, C>(p, stream);
  return launch_cfg<TIn, TOut, false, true, C>(p, stream);
}

// The 256 x 256 configuration only when it still yields a workgroup per CU;
// small batched products (the Cayley VJP) go to the 128 x 128 one.
bool use_big(const GemmParams& p) {
  const int64_t tiles = (int64_t)((p.M + 255) / 256) * ((p.N + 255) / 256) * p.batch * p.ksplit;
  return p.M >= 256 && p.N >= 256 && tiles >= 256;
}

// small batched products (the Cayley VJP's b x b blocks, small grams): 64 x 64
// tiles when 128 x 128 ones would leave CUs idle. Measured on the VJP of 16
// blocks of 256 (64 tiles of 128): 39.6 -> 27.5 us; with 72 blocks (288
// tiles) the 128 tiles stay faster (57 vs 67 us).
bool use_tiny(const GemmParams& p) {
  const int64_t tiles = (int64_t)((p.M + 127) / 128) * ((p.N + 127) / 128) * p.batch * p.ksplit;
  return p.M <= 256 && p.N <= 256 && p.K <= 1024 && tiles < 256;
}

}  // namespace

int gemm_k_tile(DType in) { return in == DType::BF16 ? 64 : 32; }

int gemm_tile_m(DType in, int M, int N) {
  if (in == DType::BF16) return (M >= 256 && N >= 256) ? 256 : 128;
  return M >= 128 ? 128 : 64;
}

hipError_t launch_gemm(DType in, DType out, bool a_kmajor, bool b_kmajor, const GemmParams& p,
                       hipStream_t stream) {
  if (p.batch <= 0 || p.M <= 0 || p.N <= 0 || p.ksplit <= 0) return hipSuccess;
  if (in == DType::BF16) {
    const bool big = use_big(p);
    if (!big && use_tiny(p)) {
      if (out == DType::BF16) return launch_layout<bf16_t, bf16_t, TinyBf16>(a_kmajor, b_kmajor, p, stream);
      return launch_layout<bf16_t, float, TinyBf16>(a_kmajor, b_kmajor, p, stream);
    }
    if (out == DType::BF16)
      return big ? launch_layout<bf16_t, bf16_t, Big>(a_kmajor, b_kmajor, p, stream)
                 : launch_layout<bf16_t, bf16_t, SmallBf16>(a_kmajor, b_kmajor, p, stream);
    return big ? launch_layout<bf16_t, float, Big>(a_kmajor, b_kmajor, p, stream)
               : launch_layout<bf16_t, float, SmallBf16>(a_kmajor, b_kmajor, p, stream);
  }
  if (out == DType::F32 && bmm32_supported(p, a_kmajor, b_kmajor)) return launch_bmm32(p, stream);
  if (p.C_act || p.C2_act) return hipErrorInvalidValue;  // only bmm32 writes the bf16 copies
  if (out == DType::F32)
    return p.M >= 128 ? launch_layout<float, float, MidF32>(a_kmajor, b_kmajor, p, stream)
                      : launch_layout<float, float, SmallF32>(a_kmajor, b_kmajor, p, stream);
  return hipErrorInvalidValue;
}

}  // namespace poetx
