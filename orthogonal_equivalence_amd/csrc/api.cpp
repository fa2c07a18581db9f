// C ABI of libpoetx: argument validation, workspace planning and the order
// of kernel launches for the POET-X linear layer. Declarations and the
// contract of every entry point are in include/poetx.h.
//
// Validation touches no HIP API, so every argument error is reported before
// anything is enqueued (and can be exercised without a GPU).
#include "poetx.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "kernels.h"

using poetx::DType;
using poetx::GemmParams;

namespace {

constexpr int kMaxBlock = 4096;
constexpr int64_t kMaxBatch = 65535;  // grid.y limit of the batched launches
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t act_size(int act) { return act == POETX_BF16 ? 2 : 4; }
int act_vec(int act) { return act == POETX_BF16 ? 8 : 4; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;
};
Range range_of(const void* p, size_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Checks shape, dtype and alignment fields of a descriptor.
int check_desc(const poetx_linear_desc* d) {
  if (!d) return POETX_ERR_NULL;
  if (d->act != POETX_F32 && d->act != POETX_BF16) return POETX_ERR_DTYPE;
  if (d->tokens < 1 || d->d_in < 1 || d->d_out < 1) return POETX_ERR_SHAPE;
  if (d->tokens > INT32_MAX || d->d_in > INT32_MAX || d->d_out > INT32_MAX) return POETX_ERR_SHAPE;
  if (d->b_in < 1 || d->b_out < 1 || d->b_in > kMaxBlock || d->b_out > kMaxBlock) return POETX_ERR_SHAPE;
  if (d->b_in > d->d_in || d->b_out > d->d_out) return POETX_ERR_SHAPE;
  if (ceil_div(d->d_in, d->b_in) > kMaxBatch || ceil_div(d->d_out, d->b_out) > kMaxBatch) return POETX_ERR_SHAPE;
  if (d->n_events < 0 || (d->n_events > 0 && !d->events)) return POETX_ERR_NULL;
  if ((d->flags & ~(POETX_RECOMPUTE_Z | POETX_CAYLEY_NEUMANN | POETX_SAVED_Y)) != 0 ||
      d->reserved != 0)
    return POETX_ERR_SHAPE;
  if ((d->perm_in == nullptr) != (d->perm_out == nullptr)) return POETX_ERR_NULL;
  // Z = Y R needs exactly orthogonal blocks and y in block order
  if ((d->flags & POETX_SAVED_Y) &&
      ((d->flags & (POETX_RECOMPUTE_Z | POETX_CAYLEY_NEUMANN)) || d->perm_in != nullptr))
    return POETX_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(d->perm_in) & 3) || (reinterpret_cast<uintptr_t>(d->perm_out) & 3))
    return POETX_ERR_ALIGN;
  // INT8 weight codes are widened 8 at a time
  if (d->w_scale && ((reinterpret_cast<uintptr_t>(d->w_scale) & 3) || d->d_in % 8))
    return POETX_ERR_ALIGN;
  const int v = act_vec(d->act);
  if (d->d_in % v || d->d_out % v || d->b_in % v || d->b_out % v) return POETX_ERR_ALIGN;
  return POETX_OK;
}

// ---------------------------------------------------------------- workspace
bool recompute_z(const poetx_linear_desc* d) { return (d->flags & POETX_RECOMPUTE_Z) != 0; }
bool neumann(const poetx_linear_desc* d) { return (d->flags & POETX_CAYLEY_NEUMANN) != 0; }
bool saved_y(const poetx_linear_desc* d) { return (d->flags & POETX_SAVED_Y) != 0; }
bool permuted(const poetx_linear_desc* d) { return d->perm_in != nullptr; }
bool int8_weight(const poetx_linear_desc* d) { return d->w_scale != nullptr; }
size_t weight_bytes(const poetx_linear_desc* d) {
  return (size_t)d->d_out * d->d_in * (int8_weight(d) ? 1 : act_size(d->act));
}

// An INT8 layer widens its codes to the activation type in chunks of weight
// rows (the forward's product, whose output columns they are) or weight
// columns (the backward's, likewise), so the transient act-type copy holds a
// fraction of the weight. A forward chunk is enough for about two rounds of
// 256 x 256 output tiles of the dense kernel (256 workgroups at 256 tokens
// per tile row), a backward chunk for one: the forward's tiles are short
// (K = d_in), so each launch's start costs more there (measured at 8192
// tokens of the 8B MLP-up layer: one round per forward chunk, 7 launches,
// added ~25 us to its 0.79 ms). int8_chunk: the nominal chunk (a multiple of
// 256, or the whole width when that is smaller); next_chunk: the chunk at c0,
// which also takes a remainder narrower than 256 (so no chunk but a whole
// narrow width is under 256 wide, and the dense kernel takes every chunk
// that the whole product would have); int8_chunk_max: the widest chunk.
constexpr int kFwdChunkRounds = 2, kBwdChunkRounds = 1;
int64_t int8_chunk(int64_t tokens, int64_t width, int rounds) {
  const int64_t tile_rows = ceil_div(tokens, 256);
  const int64_t c = std::max<int64_t>(1, 256 * rounds / tile_rows) * 256;
  return std::min(c, width);
}
int64_t next_chunk(int64_t c0, int64_t width, int64_t cw) {
  const int64_t rem = width - c0;
  return (rem <= cw || rem - cw < 256) ? rem : cw;
}
int64_t int8_chunk_max(int64_t tokens, int64_t width, int rounds) {
  const int64_t cw = int8_chunk(tokens, width, rounds);
  int64_t widest = 0;
  for (int64_t c0 = 0, cn; c0 < width; c0 += cn) {
    cn = next_chunk(c0, width, cw);
    widest = std::max(widest, cn);
  }
  return widest;
}

struct FwdPlan {
  size_t u_off, z_off, xp_off, yp_off, inv_off, wq_off, rs_off, sb_off, total;
};

// Whether the forward runs the R-apply in the dense kernel's epilogue: bf16
// with 256 x 256 R blocks, every 256-column output tile being one block.
bool fwd_fuses_r(const poetx_linear_desc* d) {
  const int64_t N = d->tokens, n = d->d_in, m = d->d_out;
  return d->act == POETX_BF16 && d->b_out == 256 && m % 256 == 0 &&
         poetx::dense_fused_r_supported(N, m, n, n, n, m, m);
}

// Bytes of the super-block buffer (block-diagonal 128 x 128 super blocks of
// b = 32 or 64 blocks, for the b = 128 streaming kernels): one side at a
// time, so the larger of the two.
size_t superblock_bytes(const poetx_linear_desc* d) {
  const DType t = d->act == POETX_BF16 ? DType::BF16 : DType::F32;
  size_t n = 0;
  if (int S = poetx::superblock_size(t, d->d_in, d->b_in)) n = std::max(n, (size_t)d->d_in * S);
  if (int S = poetx::superblock_size(t, d->d_out, d->b_out)) n = std::max(n, (size_t)d->d_out * S);
  return n * act_size(d->act);
}
FwdPlan plan_fwd(const poetx_linear_desc* d) {
  FwdPlan p;
  const size_t es = act_size(d->act);
  p.u_off = 0;
  size_t off = align_up((size_t)d->tokens * d->d_in * es);
  p.z_off = off;  // Z lives here only when it is not kept, and is formed
  if (recompute_z(d) || (saved_y(d) && !fwd_fuses_r(d)))
    off += align_up((size_t)d->tokens * d->d_out * es);
  // with permutations: the gathered x, Y before its scatter, the inverse map
  p.xp_off = p.yp_off = p.inv_off = off;
  if (permuted(d)) {
    p.xp_off = off; off += align_up((size_t)d->tokens * d->d_in * es);
    p.yp_off = off; off += align_up((size_t)d->tokens * d->d_out * es);
    p.inv_off = off; off += align_up((size_t)d->d_out * 4);
  }
  // INT8 weight: one chunk of widened code rows and the column-scaled R blocks
  p.wq_off = p.rs_off = off;
  if (int8_weight(d)) {
    p.wq_off = off;
    off += align_up((size_t)int8_chunk_max(d->tokens, d->d_out, kFwdChunkRounds) * d->d_in * es);
    p.rs_off = off; off += align_up((size_t)ceil_div(d->d_out, d->b_out) * d->b_out * d->b_out * es);
  }
  p.sb_off = off; off += align_up(superblock_bytes(d));
  p.total = off;
  return p;
}

struct SplitK {
  int nsplit, kchunk;
};
// Splits the token reduction of a gram so the launch fills the chip (about
// 256 workgroups of the 256 x 256 tile, 1024 of the smaller ones), with at
// least 256 tokens per split.
SplitK choose_split(int64_t nblocks, int b, int64_t d, int64_t tokens, DType in) {
  if (poetx::blockgram_supported(in, d, b)) {
    // streaming gram: one round of about 256 workgroups
    int64_t s = std::max<int64_t>(1, 256 / (nblocks * poetx::blockgram_wg_per_block(b)));
    s = std::min<int64_t>(s, std::max<int64_t>(1, tokens / 256));
    const int64_t chunk = ceil_div(ceil_div(tokens, s), 64) * 64;
    SplitK r;
    r.kchunk = (int)chunk;
    r.nsplit = (int)ceil_div(tokens, chunk);
    return r;
  }
  const int mt = poetx::gemm_tile_m(in, b, b);
  const int kt = poetx::gemm_k_tile(in);
  const int64_t tiles = nblocks * ceil_div(b, mt) * ceil_div(b, mt);
  const int64_t target = mt >= 256 ? 256 : 1024;
  int64_t s = std::max<int64_t>(1, ceil_div(target, tiles));
  s = std::min<int64_t>(s, std::max<int64_t>(1, tokens / 256));
  int64_t chunk = ceil_div(ceil_div(tokens, s), kt) * kt;
  SplitK r;
  r.kchunk = (int)chunk;
  r.nsplit = (int)ceil_div(tokens, chunk);
  return r;
}

struct BwdPlan {
  size_t gz, gu, partR, partP, GR, GP, TR, TP, MR, MP, gyp, xp, inv, wq, rs, sb, total;
  SplitK sR, sP;
  int subR, subP;  // blocks per super block of the grams (1: none)
};
BwdPlan plan_bwd(const poetx_linear_desc* d) {
  BwdPlan p;
  const DType in = d->act == POETX_BF16 ? DType::BF16 : DType::F32;
  const int64_t nbR = ceil_div(d->d_out, d->b_out), nbP = ceil_div(d->d_in, d->b_in);
  const size_t bbR = (size_t)d->b_out * d->b_out * 4, bbP = (size_t)d->b_in * d->b_in * 4;
  // the grams of b = 32 / 64 blocks run as grams of their 128 x 128 super
  // blocks, whose diagonal pieces the reduction keeps
  const int SR = poetx::superblock_size(in, d->d_out, d->b_out);
  const int SP = poetx::superblock_size(in, d->d_in, d->b_in);
  p.subR = SR ? SR / d->b_out : 1;
  p.subP = SP ? SP / d->b_in : 1;
  p.sR = SR ? choose_split(d->d_out / SR, SR, d->d_out, d->tokens, in)
            : choose_split(nbR, d->b_out, d->d_out, d->tokens, in);
  p.sP = SP ? choose_split(d->d_in / SP, SP, d->d_in, d->tokens, in)
            : choose_split(nbP, d->b_in, d->d_in, d->tokens, in);
  size_t off = 0;
  p.gz = off; off += align_up((size_t)d->tokens * d->d_out * act_size(d->act));
  p.gu = off; off += align_up((size_t)d->tokens * d->d_in * act_size(d->act));
  p.partR = off; off += align_up((size_t)p.sR.nsplit * nbR * bbR * p.subR);
  p.partP = off; off += align_up((size_t)p.sP.nsplit * nbP * bbP * p.subP);
  p.GR = off; off += align_up(nbR * bbR);
  p.GP = off; off += align_up(nbP * bbP);
  p.TR = off; off += align_up(nbR * bbR);
  p.TP = off; off += align_up(nbP * bbP);
  p.MR = off; off += align_up(nbR * bbR);
  p.MP = off; off += align_up(nbP * bbP);
  // with permutations: gathered g_y, gathered x (then g_X before its
  // scatter), the inverse map of perm_in
  p.gyp = p.xp = p.inv = off;
  if (permuted(d)) {
    p.gyp = off; off += align_up((size_t)d->tokens * d->d_out * act_size(d->act));
    p.xp = off; off += align_up((size_t)d->tokens * d->d_in * act_size(d->act));
    p.inv = off; off += align_up((size_t)d->d_in * 4);
  }
  p.wq = p.rs = off;
  if (int8_weight(d)) {
    // one region for a chunk of widened code columns (B3) or code rows (the
    // recompute of Z), and, between those two uses, R's column-scaled
    // blocks (read by B1 only)
    const size_t es = act_size(d->act);
    const size_t cols = (size_t)d->d_out * int8_chunk_max(d->tokens, d->d_in, kBwdChunkRounds);
    const size_t rows =
        recompute_z(d) ? (size_t)int8_chunk_max(d->tokens, d->d_out, kFwdChunkRounds) * d->d_in : 0;
    const size_t rsb = (size_t)nbR * d->b_out * d->b_out;
    p.wq = p.rs = off;
    off += align_up(std::max({cols, rows, rsb}) * es);
  }
  p.sb = off; off += align_up(superblock_bytes(d));
  p.total = off;
  return p;
}

// ---------------------------------------------------------------- helpers
struct Stages {
  const poetx_linear_desc* d;
  hipStream_t s;
  hipError_t begin(int i) const { return mark(2 * i); }
  hipError_t end(int i) const { return mark(2 * i + 1); }
  hipError_t mark(int e) const {
    if (e + 1 > d->n_events || d->events[e] == nullptr) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(d->events[e]), s);
  }
};

// Block-diagonal product of token-major activations:
//   out[:, blk] = in[:, blk] M_blk^T (transpose) or in[:, blk] M_blk
GemmParams blockdiag_params(const void* in, const void* blocks, void* out, int64_t tokens,
                            int64_t d, int b, bool transpose_blocks, bool* b_kmajor) {
  GemmParams g;
  const int64_t nb = ceil_div(d, b);
  const int last = (int)(d - (nb - 1) * b);
  g.A = in; g.lda = d; g.sA = b;
  g.B = blocks; g.ldb = b; g.sB = (int64_t)b * b;
  g.C = out; g.ldc = d; g.sC = b;
  g.M = g.M_last = (int)tokens;
  g.N = g.K = b;
  g.N_last = g.K_last = last;
  g.batch = (int)nb;
  g.kchunk = b;
  *b_kmajor = transpose_blocks;  // M^T: B(n, k) = M[n][k]; M: B(n, k) = M[k][n]
  return g;
}

// How block_apply runs a shape: b = 32 / 64 on 128 x 128 super blocks
// through the b = 128 streaming kernel, b >= 512 on the batched dense kernel
// when the streaming kernel would underfill, b = 128 / 256 / 512 on the
// streaming kernel, else on the batched GEMM.
enum class ApplyPath { Super, DenseBatched, Stream, Gemm };
ApplyPath apply_path(DType t, int64_t tokens, int64_t d, int b) {
  if (poetx::superblock_size(t, d, b)) return ApplyPath::Super;
  const bool streaming = poetx::blockapply_supported(t, d, b);
  // Blocks of 512 and more: the batched dense kernel, one 256 x 256 output
  // tile of one block per workgroup, all blocks in one launch. For b = 512
  // the streaming kernel is faster once each of its workgroups covers more
  // than 512 tokens: with K = 512 the dense kernel's tile fill and store take
  // about as long as its 16 K steps (measured: 16384 tokens of d = 14336,
  // 306 us streaming against 385 us dense; 8192 tokens of d = 4096, 54 us
  // streaming against 48 us dense).
  if (t == DType::BF16 && b >= 512 && b % 256 == 0 && d % b == 0 &&
      poetx::dense_supported(tokens, b, b, d, b, d) &&
      (!streaming || poetx::blockapply_tokens_per_workgroup(tokens, d, b) <= 512))
    return ApplyPath::DenseBatched;
  return streaming ? ApplyPath::Stream : ApplyPath::Gemm;
}

// Whether block_apply can write its output in the tiled layout for this shape
// (a streaming kernel and whole 256-token panels).
bool apply_tiles(DType t, int64_t tokens, int64_t d, int b) {
  const ApplyPath a = apply_path(t, tokens, d, b);
  return tokens % poetx::kTileRows == 0 && (a == ApplyPath::Super || a == ApplyPath::Stream);
}

// out[:, blk] = in[:, blk] M_blk^T (transpose) or in[:, blk] M_blk, along
// apply_path; out_tiled (only where apply_tiles holds) writes out in the
// tiled layout.
hipError_t block_apply(DType t, const void* in, const void* blocks, void* out, int64_t tokens,
                       int64_t d, int b, bool transpose, hipStream_t s, void* super_ws,
                       bool out_tiled = false) {
  const ApplyPath a = apply_path(t, tokens, d, b);
  if (out_tiled && !apply_tiles(t, tokens, d, b)) return hipErrorInvalidValue;
  switch (a) {
    case ApplyPath::Super: {
      // the blocks placed on the diagonals of 128 x 128 super blocks (zeros
      // elsewhere) and applied by the b = 128 streaming kernel
      const int S = poetx::superblock_size(t, d, b);
      hipError_t e = poetx::launch_superblocks(blocks, d / b, b, S, super_ws, s);
      if (e != hipSuccess) return e;
      return poetx::launch_blockapply(in, super_ws, out, tokens, d, S, transpose, out_tiled, s);
    }
    case ApplyPath::DenseBatched:
      return poetx::launch_dense_batched(in, blocks, out, tokens, b, b, d, b, d, transpose, d / b,
                                         b, (int64_t)b * b, b, s);
    case ApplyPath::Stream:
      return poetx::launch_blockapply(in, blocks, out, tokens, d, b, transpose, out_tiled, s);
    case ApplyPath::Gemm:
      break;
  }
  bool bk;
  GemmParams g = blockdiag_params(in, blocks, out, tokens, d, b, transpose, &bk);
  return poetx::launch_gemm(t, t, true, bk, g, s);
}

// Gram of token-major activations: part[s][blk] = a[:, blk]^T c[:, blk]
GemmParams gram_params(const void* a, const void* c, float* part, int64_t tokens, int64_t d, int b,
                       SplitK sk) {
  GemmParams g;
  const int64_t nb = ceil_div(d, b);
  const int last = (int)(d - (nb - 1) * b);
  g.A = a; g.lda = d; g.sA = b;
  g.B = c; g.ldb = d; g.sB = b;
  g.C = part; g.ldc = b; g.sC = (int64_t)b * b;
  g.M = g.N = b;
  g.M_last = g.N_last = last;
  g.K = g.K_last = (int)tokens;
  g.batch = (int)nb;
  g.ksplit = sk.nsplit;
  g.kchunk = sk.kchunk;
  g.sC_split = nb * (int64_t)b * b;
  return g;
}

// part[s][blk] = a[:, blk]^T c[:, blk] over split s, on the streaming kernel
// when it supports the shape, else on the batched split-K GEMM.
hipError_t block_gram(DType t, const void* a, const void* c, float* part, int64_t tokens, int64_t d,
                      int b, SplitK sk, hipStream_t s) {
  if (const int S = poetx::superblock_size(t, d, b))  // grams of the 128 x 128 super blocks
    return poetx::launch_blockgram(a, c, part, tokens, d, S, sk.nsplit, sk.kchunk, s);
  if (poetx::blockgram_supported(t, d, b))
    return poetx::launch_blockgram(a, c, part, tokens, d, b, sk.nsplit, sk.kchunk, s);
  GemmParams g = gram_params(a, c, part, tokens, d, b, sk);
  return poetx::launch_gemm(t, DType::F32, false, false, g, s);
}

// Whether dense() runs on the persistent dense kernel, which can read A in
// the tiled layout.
bool dense_direct(DType t, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc) {
  return t == DType::BF16 && poetx::dense_supported(M, N, K, lda, ldb, ldc);
}

// A dense W0 product C[M][N] = A[M][K] B(n, k) (B(n, k) = B[n][k] when
// b_kmajor, else B[k][n]): the persistent direct-to-LDS bf16 kernel when the
// shape allows it, else the general GEMM. a_tiled, b_tiled (only where
// dense_direct holds): A, a K-major B in the tiled layout.
hipError_t dense(DType t, const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                 int64_t lda, int64_t ldb, int64_t ldc, bool b_kmajor, hipStream_t s,
                 bool a_tiled = false, bool b_tiled = false) {
  if (dense_direct(t, M, N, K, lda, ldb, ldc))
    return poetx::launch_dense(A, B, C, M, N, K, lda, ldb, ldc, b_kmajor, a_tiled, b_tiled, s);
  if (a_tiled || b_tiled) return hipErrorInvalidValue;
  GemmParams g;
  g.A = A; g.lda = lda;
  g.B = B; g.ldb = ldb;
  g.C = C; g.ldc = ldc;
  g.M = g.M_last = (int)M; g.N = g.N_last = (int)N; g.K = g.K_last = (int)K;
  g.kchunk = (int)K;
  return poetx::launch_gemm(t, t, true, b_kmajor, g, s);
}

// The forward's dense product Z = U W^T (W = W0, or the INT8 codes q), and
// with R (256 x 256 blocks, fused) also Y = Z blockdiag(R)^T in the same
// launches (then Z may be NULL: Y alone is written). With INT8 codes the output columns go in chunks (next_chunk):
// each chunk's code rows widened into Wq, then its columns of Z (and Y);
// Wq in the tiled layout when the dense kernel reads it and the chunk's
// shape allows.
hipError_t dense_forward(DType t, const poetx_linear_desc* d, const void* U, const void* W0,
                         void* Wq, void* Z, const void* R, void* Y, bool u_tiled, hipStream_t s) {
  const int64_t N = d->tokens, n = d->d_in, m = d->d_out;
  const size_t es = act_size(d->act);
  const bool q8 = int8_weight(d);
  const int64_t cw = q8 ? int8_chunk(N, m, kFwdChunkRounds) : m;
  for (int64_t c0 = 0, cn; c0 < m; c0 += cn) {
    cn = next_chunk(c0, m, cw);
    const void* Wc = static_cast<const char*>(W0) + c0 * n * es;
    const bool w_tiled = q8 && dense_direct(t, N, cn, n, n, n, m) &&
                         cn % poetx::kTileRows == 0 && n % poetx::kTileCols == 0;
    hipError_t e;
    if (q8) {
      e = poetx::launch_widen_codes(t, static_cast<const int8_t*>(W0) + c0 * n, cn, n, n, Wq,
                                    w_tiled, s);
      if (e != hipSuccess) return e;
      Wc = Wq;
    }
    void* Zc = Z ? static_cast<char*>(Z) + c0 * es : nullptr;  // (no Z: fused only)
    if (R)  // (c0 and cn are multiples of 256 here: m is, and so is the nominal chunk)
      e = poetx::launch_dense_fused_r(U, Wc, Zc, N, cn, n, n, n, m,
                                      static_cast<const char*>(R) + (c0 / 256) * 256 * 256 * es,
                                      static_cast<char*>(Y) + c0 * es, m, u_tiled, w_tiled, s);
    else
      e = dense(t, U, Wc, Zc, N, cn, n, n, n, m, true, s, u_tiled, w_tiled);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The backward's dense product g_U = g_Z W (B(n, k) = W[k][n]); with INT8
// codes in chunks of output columns, each chunk's code columns widened into
// Wq (d_out rows of cn).
hipError_t dense_backward(DType t, const poetx_linear_desc* d, const void* gZ, const void* W0,
                          void* Wq, void* gU, bool gz_tiled, hipStream_t s) {
  const int64_t N = d->tokens, n = d->d_in, m = d->d_out;
  const size_t es = act_size(d->act);
  const bool q8 = int8_weight(d);
  const int64_t cw = q8 ? int8_chunk(N, n, kBwdChunkRounds) : n;
  for (int64_t c0 = 0, cn; c0 < n; c0 += cn) {
    cn = next_chunk(c0, n, cw);
    const void* B = static_cast<const char*>(W0) + c0 * es;
    int64_t ldb = n;
    hipError_t e;
    if (q8) {
      e = poetx::launch_widen_codes(t, static_cast<const int8_t*>(W0) + c0, m, n, cn, Wq, false,
                                    s);
      if (e != hipSuccess) return e;
      B = Wq;
      ldb = cn;
    }
    e = dense(t, gZ, B, static_cast<char*>(gU) + c0 * es, N, cn, m, m, ldb, n, false, s, gz_tiled);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Cayley VJP of every block: M = 1/2 (R^T + I) G (R^T + I), packed as
// g_theta(i, j) = M[i][j] - M[j][i]. Computed as T = G R^T + G
// (= G (R^T + I): both operands and the addend read in their stored order)
// and M = 1/2 (R^T T + T), whose A operand R^T the GEMM reads column-wise
// (its MN-major loader). A set whose gram was formed from Y (POETX_SAVED_Y:
// G = G' R with G' = g_Y^T Y) instead takes T = G' R + G' (= G (R^T + I),
// since R R^T = I), the GEMM reading R row-wise; the second product is the
// same. When a second block set of the same size is given, both run in the
// same launches (the first product in two when their forms differ).
//
// float32 activations: float32 products throughout. bf16 activations: G and
// T are rounded to bf16 and both products run on bf16 MFMA with float32
// accumulation (R^T T in float32; the 1/2 T term is added in float32 by the
// pack), which adds about 2^-8 relative error to a gradient already formed
// from bf16 activations.
struct VjpSet {
  const void* G;       // float32 or bf16 (the activation type)
  const float* R;      // float32 blocks
  const void* R_act;   // activation-type blocks
  void* T;             // same type as G
  float* M;            // M (float32) or 1/2 R^T T (bf16 path)
  float* g_theta;
  int64_t d;
  bool from_y;         // G holds G' = g_Y^T Y (POETX_SAVED_Y)
};
hipError_t cayley_vjp(DType t, const VjpSet& a, const VjpSet* b2, int b, hipStream_t s) {
  const int64_t nb1 = ceil_div(a.d, b);
  const int64_t nb2 = b2 ? ceil_div(b2->d, b) : 0;
  const int64_t bb = (int64_t)b * b;
  const bool lowp = t == DType::BF16;
  GemmParams g;
  // T = G R^T + G: A = G (K-major), B(n, k) = R[n][k] (K-major), addend G;
  // T = G' R + G': B(n, k) = R[k][n] (N-major)
  g.A = a.G; g.lda = b; g.sA = bb;
  g.B = lowp ? a.R_act : a.R; g.ldb = b; g.sB = bb;
  g.C = a.T; g.ldc = b; g.sC = bb;
  g.D = a.G; g.ldd = b; g.sD = bb;
  g.M = g.N = g.K = g.M_last = g.N_last = g.K_last = b;
  g.batch = (int)nb1;
  g.kchunk = b;
  g.alpha = 1.0f; g.beta = 1.0f;
  hipError_t e;
  if (b2 && b2->from_y == a.from_y) {
    g.batch = (int)(nb1 + nb2);
    g.batch_split = (int)nb1;
    g.A2 = b2->G; g.B2 = lowp ? b2->R_act : b2->R; g.C2 = b2->T; g.D2 = b2->G;
    if ((e = poetx::launch_gemm(t, t, true, !a.from_y, g, s)) != hipSuccess) return e;
  } else {
    if ((e = poetx::launch_gemm(t, t, true, !a.from_y, g, s)) != hipSuccess) return e;
    if (b2) {
      GemmParams g2 = g;
      g2.A = b2->G; g2.B = lowp ? b2->R_act : b2->R; g2.C = b2->T; g2.D = b2->G;
      g2.batch = (int)nb2;
      if ((e = poetx::launch_gemm(t, t, true, !b2->from_y, g2, s)) != hipSuccess) return e;
    }
  }
  // M = 1/2 (R^T T + T): A(m, k) = R[k][m] (MN-major), B(n, k) = T[k][n]; in
  // the bf16 path the GEMM writes 1/2 R^T T and the pack adds 1/2 T
  g.batch = (int)(nb1 + nb2);
  if (b2) g.batch_split = (int)nb1;
  g.A = lowp ? a.R_act : a.R; g.B = a.T; g.C = a.M;
  g.alpha = 0.5f;
  g.D = lowp ? nullptr : a.T; g.beta = lowp ? 0.0f : 0.5f;
  if (b2) {
    g.A2 = lowp ? b2->R_act : b2->R; g.B2 = b2->T; g.C2 = b2->M; g.D2 = lowp ? nullptr : b2->T;
  }
  e = poetx::launch_gemm(t, DType::F32, false, false, g, s);
  if (e != hipSuccess) return e;
  const poetx::PackSet p1{a.M, lowp ? a.T : nullptr, nb1, (int)(a.d - (nb1 - 1) * b), a.g_theta};
  if (!b2) return poetx::launch_pack_skew_grad(p1, nullptr, 0.5f, b, 1.0f, s);
  const poetx::PackSet p2{b2->M, lowp ? b2->T : nullptr, nb2, (int)(b2->d - (nb2 - 1) * b),
                          b2->g_theta};
  return poetx::launch_pack_skew_grad(p1, &p2, 0.5f, b, 1.0f, s);
}

// VJP of the truncated Cayley-Neumann series R = I + 2 (Q + Q^2 + Q^3 + Q^4)
// for every block, float32 throughout for float32 activations (bf16 mode:
// cnp_vjp_bf16 below; the factored form is derived in cnp.hip):
//   Q2 = Q Q -> w1;  Tt = Q2 - Q -> w2;  Tbar = 2 G Q2 + 2 G -> w3;
//   Nbar = 2 Tt G -> w1;  Ws = (Tbar + Nbar) + (Tbar + Nbar)^T -> w2;
//   X = Tbar - Ws Q -> w1;  g_theta(i, j) = X[i][j] - X[j][i].
// w1..w3 are b x b float32 scratch sets; G and Q are only read. A second
// block set of the same size shares the GEMM launches.
struct CnpVjpSet {
  const float* G;  // float32 gram (dL/dR per block)
  const float* Q;  // float32 skew blocks
  float* w1;
  float* w2;
  float* w3;
  float* g_theta;
  int64_t d;
};
hipError_t cnp_vjp(const CnpVjpSet& a, const CnpVjpSet* b2, int b, hipStream_t s) {
  const int64_t nb1 = ceil_div(a.d, b);
  const int64_t nb2 = b2 ? ceil_div(b2->d, b) : 0;
  const int64_t bb = (int64_t)b * b;
  GemmParams g;
  g.lda = g.ldb = g.ldc = g.ldd = b;
  g.sA = g.sB = g.sC = g.sD = bb;
  g.M = g.N = g.K = g.M_last = g.N_last = g.K_last = b;
  g.kchunk = b;
  g.batch = (int)(nb1 + nb2);
  if (b2) g.batch_split = (int)nb1;
  // C = alpha A B + beta D per block (A, B row-major b x b)
  auto mm = [&](const float* A1, const float* B1, float* C1, const float* D1, const float* A2,
                const float* B2, float* C2, const float* D2, float alpha, float beta) {
    g.A = A1; g.B = B1; g.C = C1; g.D = D1;
    g.A2 = A2; g.B2 = B2; g.C2 = C2; g.D2 = D2;
    g.alpha = alpha; g.beta = beta;
    return poetx::launch_gemm(DType::F32, DType::F32, true, false, g, s);
  };
  const CnpVjpSet z{};
  const CnpVjpSet& c = b2 ? *b2 : z;
  hipError_t e;
  if ((e = mm(a.Q, a.Q, a.w1, nullptr, c.Q, c.Q, c.w1, nullptr, 1.0f, 0.0f)) != hipSuccess) return e;
  if ((e = poetx::launch_sub(a.w1, a.Q, a.w2, nb1 * bb, s)) != hipSuccess) return e;
  if (b2 && (e = poetx::launch_sub(c.w1, c.Q, c.w2, nb2 * bb, s)) != hipSuccess) return e;
  if ((e = mm(a.G, a.w1, a.w3, a.G, c.G, c.w1, c.w3, c.G, 2.0f, 2.0f)) != hipSuccess) return e;
  if ((e = mm(a.w2, a.G, a.w1, nullptr, c.w2, c.G, c.w1, nullptr, 2.0f, 0.0f)) != hipSuccess) return e;
  if ((e = poetx::launch_sym_sum(a.w3, a.w1, a.w2, nb1, b, s)) != hipSuccess) return e;
  if (b2 && (e = poetx::launch_sym_sum(c.w3, c.w1, c.w2, nb2, b, s)) != hipSuccess) return e;
  if ((e = mm(a.w2, a.Q, a.w1, a.w3, c.w2, c.Q, c.w1, c.w3, -1.0f, 1.0f)) != hipSuccess) return e;
  const poetx::PackSet p1{a.w1, nullptr, nb1, (int)(a.d - (nb1 - 1) * b), a.g_theta};
  if (!b2) return poetx::launch_pack_skew_grad(p1, nullptr, 0.0f, b, 1.0f, s);
  const poetx::PackSet p2{c.w1, nullptr, nb2, (int)(c.d - (nb2 - 1) * b), c.g_theta};
  return poetx::launch_pack_skew_grad(p1, &p2, 0.0f, b, 1.0f, s);
}

// The series VJP for bf16 activations: the same steps with bf16 operands
// and float32 accumulation (as the exact map's VJP in bf16 mode), G the
// bf16 reduced gram:
//   Qb = bf16(Q);  Q2 = Qb Qb;  Tt = Q2 - Q;  Tbar = 2 G Q2 + 2 G;
//   Nbar = 2 Tt G;  Ws = (Tbar + Nbar) + (Tbar + Nbar)^T;  X' = -Ws Qb,
// all bf16 but X' (float32); the pack then forms (X' + Tbar) - (X' + Tbar)^T,
// X' + Tbar being X. Buffers (each [nblocks][b][b], regions of the
// backward's workspace that are free by then): Qb in the upper half of the
// gram's region, Q2 and Tt in w1 (later X'), Tbar and Nbar in w2, Ws in w3.
struct CnpVjpBf16Set {
  const void* G;   // bf16 gram, in the lower half of its float32-sized region
  const float* Q;  // float32 skew blocks
  float* w1;
  float* w2;
  float* w3;
  float* g_theta;
  int64_t d;
};
hipError_t cnp_vjp_bf16(const CnpVjpBf16Set& a, const CnpVjpBf16Set* b2, int b, hipStream_t s) {
  const int64_t nb1 = ceil_div(a.d, b);
  const int64_t nb2 = b2 ? ceil_div(b2->d, b) : 0;
  const int64_t bb = (int64_t)b * b;
  const CnpVjpBf16Set z{};
  const CnpVjpBf16Set& c = b2 ? *b2 : z;
  // bf16 views: element offset e of a float32-sized region, in bf16 elements
  auto half = [](const void* base, int64_t e) {
    return static_cast<void*>(const_cast<char*>(static_cast<const char*>(base)) + 2 * e);
  };
  void* Qb1 = half(a.G, nb1 * bb);
  void* Qb2 = b2 ? half(c.G, nb2 * bb) : nullptr;
  void* Q2_1 = a.w1;
  void* Q2_2 = c.w1;
  void* Tt1 = half(a.w1, nb1 * bb);
  void* Tt2 = b2 ? half(c.w1, nb2 * bb) : nullptr;
  void* Tb1 = a.w2;
  void* Tb2 = c.w2;
  void* Nb1 = half(a.w2, nb1 * bb);
  void* Nb2 = b2 ? half(c.w2, nb2 * bb) : nullptr;
  GemmParams g;
  g.lda = g.ldb = g.ldc = g.ldd = b;
  g.sA = g.sB = g.sC = g.sD = bb;
  g.M = g.N = g.K = g.M_last = g.N_last = g.K_last = b;
  g.kchunk = b;
  g.batch = (int)(nb1 + nb2);
  if (b2) g.batch_split = (int)nb1;
  // C = alpha A B + beta D per block (A, B row-major b x b, bf16)
  auto mm = [&](DType out, const void* A1, const void* B1, void* C1, const void* D1, const void* A2,
                const void* B2, void* C2, const void* D2, float alpha, float beta) {
    g.A = A1; g.B = B1; g.C = C1; g.D = D1;
    g.A2 = A2; g.B2 = B2; g.C2 = C2; g.D2 = D2;
    g.alpha = alpha; g.beta = beta;
    return poetx::launch_gemm(DType::BF16, out, true, false, g, s);
  };
  hipError_t e;
  if ((e = poetx::launch_sub_to_bf16(DType::F32, a.Q, nullptr, Qb1, nb1 * bb, c.Q, nullptr, Qb2,
                                     nb2 * bb, s)) != hipSuccess)
    return e;
  if ((e = mm(DType::BF16, Qb1, Qb1, Q2_1, nullptr, Qb2, Qb2, Q2_2, nullptr, 1.0f, 0.0f)) != hipSuccess)
    return e;
  if ((e = poetx::launch_sub_to_bf16(DType::BF16, Q2_1, a.Q, Tt1, nb1 * bb, Q2_2, c.Q, Tt2,
                                     nb2 * bb, s)) != hipSuccess)
    return e;
  if ((e = mm(DType::BF16, a.G, Q2_1, Tb1, a.G, c.G, Q2_2, Tb2, c.G, 2.0f, 2.0f)) != hipSuccess) return e;
  if ((e = mm(DType::BF16, Tt1, a.G, Nb1, nullptr, Tt2, c.G, Nb2, nullptr, 2.0f, 0.0f)) != hipSuccess)
    return e;
  if ((e = poetx::launch_sym_sum_bf16(Tb1, Nb1, a.w3, nb1, Tb2, Nb2, c.w3, nb2, b, s)) != hipSuccess)
    return e;
  if ((e = mm(DType::F32, a.w3, Qb1, a.w1, nullptr, c.w3, Qb2, c.w1, nullptr, -1.0f, 0.0f)) != hipSuccess)
    return e;
  const poetx::PackSet p1{a.w1, Tb1, nb1, (int)(a.d - (nb1 - 1) * b), a.g_theta};
  if (!b2) return poetx::launch_pack_skew_grad(p1, nullptr, 1.0f, b, 1.0f, s);
  const poetx::PackSet p2{c.w1, Tb2, nb2, (int)(c.d - (nb2 - 1) * b), c.g_theta};
  return poetx::launch_pack_skew_grad(p1, &p2, 1.0f, b, 1.0f, s);
}

int hip_status(hipError_t e) { return e == hipSuccess ? POETX_OK : POETX_ERR_HIP; }

// The forward's host-detectable argument faults other than the workspace.
int check_fwd_args(const poetx_linear_desc* d, const void* x, const void* W0, const void* R_act,
                   const void* P_act, const void* y, const void* z_save) {
  int st = check_desc(d);
  if (st != POETX_OK) return st;
  if (!x || !W0 || !R_act || !P_act || !y) return POETX_ERR_NULL;
  if ((recompute_z(d) || saved_y(d)) ? z_save != nullptr : z_save == nullptr) return POETX_ERR_NULL;
  const void* ptrs[] = {x, W0, R_act, P_act, y, z_save};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return POETX_ERR_ALIGN;
  return POETX_OK;
}

}  // namespace

extern "C" {

int poetx_abi_version(void) { return POETX_ABI_VERSION; }

const char* poetx_status_string(int s) {
  switch (s) {
    case POETX_OK: return "ok";
    case POETX_ERR_NULL: return "null pointer argument";
    case POETX_ERR_SHAPE: return "invalid or inconsistent shape";
    case POETX_ERR_DTYPE: return "unknown dtype";
    case POETX_ERR_ALIGN: return "pointer or size breaks the alignment rule";
    case POETX_ERR_WORKSPACE: return "workspace missing or too small";
    case POETX_ERR_HIP: return "HIP runtime error";
    case POETX_ERR_ALIAS: return "output overlaps an input";
    default: return "unknown status";
  }
}

int64_t poetx_num_blocks(int64_t d, int32_t b) { return (d < 1 || b < 1) ? 0 : ceil_div(d, b); }

int64_t poetx_theta_count(int64_t d, int32_t b) {
  return (d < 1 || b < 1) ? 0 : ceil_div(d, b) * ((int64_t)b * (b - 1) / 2);
}

size_t poetx_build_workspace_size(int64_t d, int32_t b) {
  if (d < 1 || b < 1 || b > kMaxBlock || b > d) return 0;
  return align_up(poetx::cayley_workspace_floats(ceil_div(d, b), b) * sizeof(float));
}

int poetx_build_orthogonal(const float* theta, int64_t d, int32_t b, float* blocks_f32,
                           void* blocks_act, int32_t act, void* ws, size_t ws_bytes,
                           void* stream) {
  if (act != POETX_F32 && act != POETX_BF16) return POETX_ERR_DTYPE;
  if (d < 1 || b < 1 || b > kMaxBlock || b > d) return POETX_ERR_SHAPE;
  const int64_t nb = ceil_div(d, b);
  if (nb > kMaxBatch) return POETX_ERR_SHAPE;
  if (!blocks_f32 || (b > 1 && !theta) || (act == POETX_BF16 && !blocks_act)) return POETX_ERR_NULL;
  if (!aligned16(blocks_f32) || (act == POETX_BF16 && !aligned16(blocks_act))) return POETX_ERR_ALIGN;
  const size_t need = poetx_build_workspace_size(d, b);
  if (!ws || ws_bytes < need) return POETX_ERR_WORKSPACE;
  const size_t blocks_bytes = (size_t)nb * b * b * 4;
  const Range out_f32 = range_of(blocks_f32, blocks_bytes);
  const Range out_act = range_of(blocks_act, act == POETX_BF16 ? blocks_bytes / 2 : 0);
  const Range in_theta = range_of(theta, (size_t)poetx_theta_count(d, b) * 4);
  const Range r_ws = range_of(ws, need);
  // the workspace is written too, so it may not overlap theta either
  if (overlap(out_f32, in_theta) || overlap(out_f32, r_ws) || overlap(out_act, in_theta) ||
      overlap(out_act, r_ws) || overlap(out_f32, out_act) || overlap(r_ws, in_theta))
    return POETX_ERR_ALIAS;
  const int last = (int)(d - (nb - 1) * b);
  return hip_status(poetx::launch_cayley_build(theta, nb, b, last, blocks_f32, blocks_act,
                                               act == POETX_BF16 ? DType::BF16 : DType::F32,
                                               static_cast<float*>(ws),
                                               static_cast<hipStream_t>(stream)));
}

size_t poetx_build_cnp_workspace_size(int64_t d, int32_t b) {
  if (d < 1 || b < 4 || b > kMaxBlock || b > d || b % 4) return 0;
  const int64_t nb = ceil_div(d, b);
  if (nb > kMaxBatch) return 0;
  return 2 * align_up((size_t)nb * b * b * sizeof(float));
}

int poetx_build_cnp(const float* theta, int64_t d, int32_t b, float* q_f32, float* blocks_f32,
                    void* blocks_act, int32_t act, void* ws, size_t ws_bytes, void* stream) {
  if (act != POETX_F32 && act != POETX_BF16) return POETX_ERR_DTYPE;
  if (d < 1 || b < 1 || b > kMaxBlock || b > d) return POETX_ERR_SHAPE;
  const int64_t nb = ceil_div(d, b);
  if (nb > kMaxBatch) return POETX_ERR_SHAPE;
  if (b % 4) return POETX_ERR_ALIGN;
  if (!theta || !q_f32 || !blocks_f32 || (act == POETX_BF16 && !blocks_act)) return POETX_ERR_NULL;
  if (!aligned16(q_f32) || !aligned16(blocks_f32) || (act == POETX_BF16 && !aligned16(blocks_act)))
    return POETX_ERR_ALIGN;
  const size_t need = poetx_build_cnp_workspace_size(d, b);
  if (!ws || ws_bytes < need) return POETX_ERR_WORKSPACE;
  if (!aligned16(ws)) return POETX_ERR_ALIGN;
  const size_t blocks_bytes = (size_t)nb * b * b * 4;
  const Range out_q = range_of(q_f32, blocks_bytes);
  const Range out_f32 = range_of(blocks_f32, blocks_bytes);
  const Range out_act = range_of(blocks_act, act == POETX_BF16 ? blocks_bytes / 2 : 0);
  const Range in_theta = range_of(theta, (size_t)poetx_theta_count(d, b) * 4);
  const Range r_ws = range_of(ws, need);
  const Range outs[] = {out_q, out_f32, out_act};
  if (overlap(r_ws, in_theta)) return POETX_ERR_ALIAS;  // the workspace is written
  for (int i = 0; i < 3; ++i) {
    if (overlap(outs[i], in_theta) || overlap(outs[i], r_ws)) return POETX_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return POETX_ERR_ALIAS;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int last = (int)(d - (nb - 1) * b);
  const int64_t bb = (int64_t)b * b;
  float* Q2 = static_cast<float*>(ws);
  float* E = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(blocks_bytes));
  hipError_t e;
  // Q (generators past d taken as zero, so a padded block's R is identity there)
  if ((e = poetx::launch_expand_skew(theta, nb, b, last, 0.0f, 1.0f, q_f32, s)) != hipSuccess)
    return hip_status(e);
  GemmParams g;
  g.lda = g.ldb = g.ldc = g.ldd = b;
  g.sA = g.sB = g.sC = g.sD = bb;
  g.M = g.N = g.K = g.M_last = g.N_last = g.K_last = b;
  g.kchunk = b;
  g.batch = (int)nb;
  // Q2 = Q Q
  g.A = q_f32; g.B = q_f32; g.C = Q2;
  if ((e = poetx::launch_gemm(DType::F32, DType::F32, true, false, g, s)) != hipSuccess)
    return hip_status(e);
  // E = Q2 Q2 + Q2 and F = Q Q2 + Q (F into blocks_f32), one launch when the
  // two segments fit the grid
  g.beta = 1.0f;
  g.A = Q2; g.B = Q2; g.C = E; g.D = Q2;
  if (2 * nb <= kMaxBatch) {
    g.batch = (int)(2 * nb);
    g.batch_split = (int)nb;
    g.A2 = q_f32; g.B2 = Q2; g.C2 = blocks_f32; g.D2 = q_f32;
    if ((e = poetx::launch_gemm(DType::F32, DType::F32, true, false, g, s)) != hipSuccess)
      return hip_status(e);
  } else {
    if ((e = poetx::launch_gemm(DType::F32, DType::F32, true, false, g, s)) != hipSuccess)
      return hip_status(e);
    g.A = q_f32; g.B = Q2; g.C = blocks_f32; g.D = q_f32;
    if ((e = poetx::launch_gemm(DType::F32, DType::F32, true, false, g, s)) != hipSuccess)
      return hip_status(e);
  }
  // R = I + 2 (E + F), in place, and the bf16 copy
  return hip_status(poetx::launch_cnp_finish(E, blocks_f32, act == POETX_BF16 ? blocks_act : nullptr,
                                             nb, b, s));
}

int poetx_fold_weight(const void* W0, int64_t d_out, int64_t d_in, const int32_t* perm_out,
                      const int32_t* perm_in, int32_t act, void* W0_folded, void* stream) {
  if (act != POETX_F32 && act != POETX_BF16) return POETX_ERR_DTYPE;
  if (d_out < 1 || d_in < 1 || d_out > INT32_MAX || d_in > INT32_MAX) return POETX_ERR_SHAPE;
  if (!W0 || !perm_out || !perm_in || !W0_folded) return POETX_ERR_NULL;
  if (d_in % act_vec(act) || !aligned16(W0) || !aligned16(W0_folded) ||
      (reinterpret_cast<uintptr_t>(perm_out) & 3) || (reinterpret_cast<uintptr_t>(perm_in) & 3))
    return POETX_ERR_ALIGN;
  const size_t bytes = (size_t)d_out * d_in * act_size(act);
  const Range out = range_of(W0_folded, bytes);
  if (overlap(out, range_of(W0, bytes)) || overlap(out, range_of(perm_out, d_out * 4)) ||
      overlap(out, range_of(perm_in, d_in * 4)))
    return POETX_ERR_ALIAS;
  const DType t = act == POETX_BF16 ? DType::BF16 : DType::F32;
  return hip_status(poetx::launch_gather_columns(t, W0, d_in, perm_out, d_out, d_out, (int)d_in,
                                                 perm_in, W0_folded, d_in,
                                                 static_cast<hipStream_t>(stream)));
}

int poetx_quantize_weight(const void* W0, int64_t d_out, int64_t d_in, int32_t act, int8_t* q,
                          float* scale, void* stream) {
  if (act != POETX_F32 && act != POETX_BF16) return POETX_ERR_DTYPE;
  if (d_out < 1 || d_in < 1 || d_out > INT32_MAX || d_in > INT32_MAX) return POETX_ERR_SHAPE;
  if (!W0 || !q || !scale) return POETX_ERR_NULL;
  if (d_in % 8 || !aligned16(W0) || !aligned16(q) || (reinterpret_cast<uintptr_t>(scale) & 3))
    return POETX_ERR_ALIGN;
  const Range in = range_of(W0, (size_t)d_out * d_in * act_size(act));
  const Range rq = range_of(q, (size_t)d_out * d_in), rs = range_of(scale, (size_t)d_out * 4);
  if (overlap(in, rq) || overlap(in, rs) || overlap(rq, rs)) return POETX_ERR_ALIAS;
  const DType t = act == POETX_BF16 ? DType::BF16 : DType::F32;
  return hip_status(poetx::launch_quantize_rows(t, W0, d_out, (int)d_in, q, scale,
                                                static_cast<hipStream_t>(stream)));
}

size_t poetx_fwd_workspace_size(const poetx_linear_desc* d) {
  if (check_desc(d) != POETX_OK) return 0;
  return plan_fwd(d).total;
}

size_t poetx_bwd_workspace_size(const poetx_linear_desc* d) {
  if (check_desc(d) != POETX_OK) return 0;
  return plan_bwd(d).total;
}

int poetx_linear_fwd(const poetx_linear_desc* d, const void* x, const void* W0, const void* R_act,
                     const void* P_act, void* y, void* z_save, void* ws, size_t ws_bytes,
                     void* stream) {
  int st = check_fwd_args(d, x, W0, R_act, P_act, y, z_save);
  if (st != POETX_OK) return st;
  if (ws && !aligned16(ws)) return POETX_ERR_ALIGN;
  const FwdPlan plan = plan_fwd(d);
  if (!ws || ws_bytes < plan.total) return POETX_ERR_WORKSPACE;

  const size_t es = act_size(d->act);
  const int64_t N = d->tokens, n = d->d_in, m = d->d_out;
  const int64_t nbR = ceil_div(m, d->b_out), nbP = ceil_div(n, d->b_in);
  const Range r_y = range_of(y, N * m * es);
  const Range r_z = z_save ? range_of(z_save, N * m * es) : Range{0, 0};
  // written: y, z and the workspace; read: everything else
  const Range r_ws = range_of(ws, plan.total);
  const Range ins[] = {range_of(x, N * n * es), range_of(W0, weight_bytes(d)),
                       range_of(R_act, nbR * d->b_out * d->b_out * es),
                       range_of(P_act, nbP * d->b_in * d->b_in * es),
                       range_of(d->perm_in, permuted(d) ? n * 4 : 0),
                       range_of(d->perm_out, permuted(d) ? m * 4 : 0),
                       range_of(d->w_scale, int8_weight(d) ? m * 4 : 0)};
  for (const Range& r : ins)
    if (overlap(r, r_y) || overlap(r, r_z) || overlap(r, r_ws)) return POETX_ERR_ALIAS;
  if (overlap(r_y, r_z) || overlap(r_y, r_ws) || overlap(r_z, r_ws)) return POETX_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const DType t = d->act == POETX_BF16 ? DType::BF16 : DType::F32;
  char* w = static_cast<char*>(ws);
  void* U = w + plan.u_off;
  const bool fuse_r = fwd_fuses_r(d);
  // (POETX_SAVED_Y with the fused R-apply: Z is never written)
  void* Z = z_save ? z_save : (saved_y(d) && fuse_r) ? nullptr : w + plan.z_off;
  const bool perm = permuted(d);
  void* Xp = w + plan.xp_off;
  void* Yp = w + plan.yp_off;
  int32_t* inv = reinterpret_cast<int32_t*>(w + plan.inv_off);
  Stages sg{d, s};
  hipError_t e;

  // stage 5 (INT8 weight only): R's blocks with column j scaled by the row
  // scale s_j, so that Y = (U q^T) (R diag(s))^T; the codes themselves are
  // widened chunk by chunk inside stage 1
  const void* Rb = R_act;
  void* Wq = w + plan.wq_off;
  if (int8_weight(d)) {
    void* Rs = w + plan.rs_off;
    if ((e = sg.begin(5)) != hipSuccess) return hip_status(e);
    if ((e = poetx::launch_scale_block_columns(t, R_act, d->w_scale, nbR, d->b_out, m, Rs, s)) !=
        hipSuccess)
      return hip_status(e);
    if ((e = sg.end(5)) != hipSuccess) return hip_status(e);
    Rb = Rs;
  }

  // stage 3 (permutations only): X_p = X[:, perm_in], the outer P permutation
  const void* X = x;
  if (perm) {
    if ((e = sg.begin(3)) != hipSuccess) return hip_status(e);
    if ((e = poetx::launch_gather_columns(t, x, n, nullptr, N, N, (int)n, d->perm_in, Xp, n, s)) !=
        hipSuccess)
      return hip_status(e);
    if ((e = sg.end(3)) != hipSuccess) return hip_status(e);
    X = Xp;
  }

  // S2: U = X blockdiag(P)^T; U is only read by the dense kernel, so it is
  // written in the tiled layout when both kernels take it
  const bool u_tiled = dense_direct(t, N, m, n, n, n, m) && apply_tiles(t, N, n, d->b_in);
  if ((e = sg.begin(0)) != hipSuccess) return hip_status(e);
  void* SB = w + plan.sb_off;  // super blocks of b = 32 / 64 blocks
  if ((e = block_apply(t, X, P_act, U, N, n, d->b_in, true, s, SB, u_tiled)) != hipSuccess)
    return hip_status(e);
  if ((e = sg.end(0)) != hipSuccess) return hip_status(e);

  // S3: Z = U W0^T, and S4: Y = Z blockdiag(R)^T. With 256 x 256 R blocks in
  // bf16 the R-apply runs in the dense kernel's epilogue: every 256-column
  // output tile is one R block, so the tile's Z, still on the CU, is
  // multiplied by its block before it leaves (stage 1 then holds both and
  // stage 2 is empty).
  void* Yout = perm ? Yp : y;
  if ((e = sg.begin(1)) != hipSuccess) return hip_status(e);
  if ((e = dense_forward(t, d, U, W0, Wq, Z, fuse_r ? Rb : nullptr, Yout, u_tiled, s)) !=
      hipSuccess)
    return hip_status(e);
  if ((e = sg.end(1)) != hipSuccess) return hip_status(e);
  if ((e = sg.begin(2)) != hipSuccess) return hip_status(e);
  if (!fuse_r && (e = block_apply(t, Z, Rb, Yout, N, m, d->b_out, true, s, SB)) != hipSuccess)
    return hip_status(e);
  if ((e = sg.end(2)) != hipSuccess) return hip_status(e);

  // stage 4 (permutations only): y[:, perm_out[i]] = Y_p[:, i], as a gather
  // by the inverse map
  if (perm) {
    if ((e = sg.begin(4)) != hipSuccess) return hip_status(e);
    if ((e = poetx::launch_invert_permutation(d->perm_out, (int)m, inv, s)) != hipSuccess)
      return hip_status(e);
    if ((e = poetx::launch_gather_columns(t, Yp, m, nullptr, N, N, (int)m, inv, y, m, s)) !=
        hipSuccess)
      return hip_status(e);
    if ((e = sg.end(4)) != hipSuccess) return hip_status(e);
  }
  return POETX_OK;
}

int poetx_linear_fwd_noalloc(const poetx_linear_desc* d, const void* x, const void* W0,
                             const void* R_act, const void* P_act, void* y, void* z_save,
                             void* stream) {
  // every argument check that needs no HIP call comes first
  int st = check_fwd_args(d, x, W0, R_act, P_act, y, z_save);
  if (st != POETX_OK) return st;
  if (plan_fwd(d).total > (size_t)POETX_NOALLOC_SCRATCH_BYTES) return POETX_ERR_WORKSPACE;
  void* scratch = nullptr;  // this device's copy of the library's scratch array
  hipError_t e = poetx::noalloc_scratch(&scratch);
  if (e != hipSuccess) return POETX_ERR_HIP;
  return poetx_linear_fwd(d, x, W0, R_act, P_act, y, z_save, scratch,
                          (size_t)POETX_NOALLOC_SCRATCH_BYTES, stream);
}

int poetx_linear_bwd(const poetx_linear_desc* d, const void* g_y, const void* x, const void* W0,
                     const float* R_f32, const float* P_f32, const void* R_act, const void* P_act,
                     const void* z_saved, void* g_x, float* g_theta_R, float* g_theta_P, void* ws,
                     size_t ws_bytes, void* stream) {
  int st = check_desc(d);
  if (st != POETX_OK) return st;
  if (!g_y || !x || !W0 || !R_f32 || !P_f32 || !R_act || !P_act || !g_x) return POETX_ERR_NULL;
  if (recompute_z(d) ? z_saved != nullptr : z_saved == nullptr) return POETX_ERR_NULL;
  if ((d->b_out > 1 && !g_theta_R) || (d->b_in > 1 && !g_theta_P)) return POETX_ERR_NULL;
  const void* ptrs[] = {g_y, x, W0, R_f32, P_f32, R_act, P_act, z_saved, g_x, g_theta_R, g_theta_P, ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return POETX_ERR_ALIGN;
  const BwdPlan plan = plan_bwd(d);
  if (!ws || ws_bytes < plan.total) return POETX_ERR_WORKSPACE;

  const size_t es = act_size(d->act);
  const int64_t N = d->tokens, n = d->d_in, m = d->d_out;
  const int bR = d->b_out, bP = d->b_in;
  const int64_t nbR = ceil_div(m, bR), nbP = ceil_div(n, bP);
  // written: g_x, both g_theta and the workspace; read: everything else
  const Range outs[] = {range_of(g_x, N * n * es),
                        range_of(g_theta_R, (size_t)poetx_theta_count(m, bR) * 4),
                        range_of(g_theta_P, (size_t)poetx_theta_count(n, bP) * 4),
                        range_of(ws, plan.total)};
  const Range ins[] = {range_of(g_y, N * m * es), range_of(x, N * n * es),
                       range_of(W0, weight_bytes(d)), range_of(R_f32, nbR * bR * bR * 4),
                       range_of(P_f32, nbP * bP * bP * 4), range_of(R_act, nbR * bR * bR * es),
                       range_of(P_act, nbP * bP * bP * es),
                       z_saved ? range_of(z_saved, N * m * es) : Range{0, 0},
                       range_of(d->perm_in, permuted(d) ? n * 4 : 0),
                       range_of(d->perm_out, permuted(d) ? m * 4 : 0),
                       range_of(d->w_scale, int8_weight(d) ? m * 4 : 0)};
  for (const Range& o : outs) {
    for (const Range& r : ins)
      if (overlap(o, r)) return POETX_ERR_ALIAS;
  }
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return POETX_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const DType t = d->act == POETX_BF16 ? DType::BF16 : DType::F32;
  char* w = static_cast<char*>(ws);
  void* gZ = w + plan.gz;
  void* gU = w + plan.gu;
  void* SB = w + plan.sb;  // super blocks of b = 32 / 64 blocks
  float* partR = reinterpret_cast<float*>(w + plan.partR);
  float* partP = reinterpret_cast<float*>(w + plan.partP);
  float* GR = reinterpret_cast<float*>(w + plan.GR);
  float* GP = reinterpret_cast<float*>(w + plan.GP);
  float* TR = reinterpret_cast<float*>(w + plan.TR);
  float* TP = reinterpret_cast<float*>(w + plan.TP);
  float* MR = reinterpret_cast<float*>(w + plan.MR);
  float* MP = reinterpret_cast<float*>(w + plan.MP);
  const int lastR = (int)(m - (nbR - 1) * bR), lastP = (int)(n - (nbP - 1) * bP);
  // the reduced grams: the activation type, except float32 for the series
  // when its bf16 VJP does not apply (b not a multiple of 8 on either side)
  const bool cnp_bf16 = neumann(d) && t == DType::BF16 && bR % 8 == 0 && bP % 8 == 0;
  const DType gt = neumann(d) && !cnp_bf16 ? DType::F32 : t;
  Stages sg{d, s};
  hipError_t e;
#define POETX_TRY(call)                            \
  do {                                             \
    if ((e = (call)) != hipSuccess) return hip_status(e); \
  } while (0)

  // stage 8 (permutations only): g_Y and X gathered by perm_out and perm_in;
  // g_X is formed in the gathered-X buffer (free after the P gram) and
  // scattered into g_x at the end
  const bool perm = permuted(d);
  const void* gY = g_y;
  const void* X = x;
  void* gX = g_x;
  int32_t* inv = reinterpret_cast<int32_t*>(w + plan.inv);
  if (perm) {
    void* gyp = w + plan.gyp;
    void* xp = w + plan.xp;
    POETX_TRY(sg.begin(8));
    POETX_TRY(poetx::launch_gather_columns(t, g_y, m, nullptr, N, N, (int)m, d->perm_out, gyp, m, s));
    POETX_TRY(poetx::launch_gather_columns(t, x, n, nullptr, N, N, (int)n, d->perm_in, xp, n, s));
    POETX_TRY(sg.end(8));
    gY = gyp;
    X = xp;
    gX = xp;
  }

  // INT8 weight: R blocks with scaled columns, g_Z' = g_Y R diag(s),
  // g_U = g_Z' q, G_R = (g_Y^T Z_q) diag(s) with Z_q = U q^T the forward's
  // saved product (with POETX_SAVED_Y, G_R = (g_Y^T Y) R unscaled: Y carries
  // the scales). The codes are widened chunk by chunk inside stages 2 and
  // 7 into the region that holds the scaled R blocks (stage 10, made after
  // stage 7) while B1 reads them.
  void* Wq = w + plan.wq;
  const void* Rb = int8_weight(d) ? static_cast<const void*>(w + plan.rs) : R_act;
  const float* gram_scale = saved_y(d) ? nullptr : d->w_scale;
  auto scale_r = [&]() -> hipError_t {
    if (!int8_weight(d)) return hipSuccess;
    hipError_t r;
    if ((r = sg.begin(10)) != hipSuccess) return r;
    if ((r = poetx::launch_scale_block_columns(t, R_act, d->w_scale, nbR, bR, m, w + plan.rs, s)) !=
        hipSuccess)
      return r;
    return sg.end(10);
  };

  // Block size the one-pass gradient apply + gram runs at for a side (bf16,
  // b = 128 or 256, or b = 32 / 64 as 128 x 128 super blocks), 0 if none.
  auto one_pass_size = [&](int64_t dd, int bb) -> int {
    if (const int S = poetx::superblock_size(t, dd, bb)) return S;
    return poetx::blockgramapply_supported(t, dd, bb) ? bb : 0;
  };
  const int opR = one_pass_size(m, bR);
  const bool fuse_r = opR != 0;
  // g_Z is only read by B3's dense kernel, so it is written in the tiled
  // layout when both kernels take it; not when the one pass reads Z from
  // the g_Z buffer itself (POET-Xmem), since tiled stores would overwrite Z
  // that other workgroups still read
  const bool gz_tiled = dense_direct(t, N, n, m, m, n, n) && N % poetx::kTileRows == 0 &&
                        (fuse_r ? z_saved != nullptr : apply_tiles(t, N, m, bR));
  auto grad_r = [&]() -> hipError_t {  // B1: g_Z = g_Y blockdiag(R)
    hipError_t r;
    if ((r = sg.begin(0)) != hipSuccess) return r;
    if ((r = block_apply(t, gY, Rb, gZ, N, m, bR, false, s, SB, gz_tiled)) != hipSuccess) return r;
    return sg.end(0);
  };
  auto gram_r = [&](const void* Z) -> hipError_t {
    // B2: G_R[k] = g_Y[:, k]^T Z[:, k], split over tokens, then reduced
    hipError_t r;
    if ((r = sg.begin(1)) != hipSuccess) return r;
    if ((r = block_gram(t, gY, Z, partR, N, m, bR, plan.sR, s)) != hipSuccess) return r;
    if ((r = poetx::launch_split_reduce(partR, plan.sR.nsplit, nbR, bR, lastR, GR, gt, s,
                                        gram_scale, plan.subR)) != hipSuccess)
      return r;
    return sg.end(1);
  };
  // B1 and B2 in one pass over g_Y (stage 0), then the gram's reduction
  // (stage 1). Each Z element is read by the one workgroup that later writes
  // g_Z at the same place, so Z may sit in the (row-major) g_Z buffer.
  auto fused_r = [&](const void* Z) -> hipError_t {
    hipError_t r;
    int ns = 0;
    if ((r = sg.begin(0)) != hipSuccess) return r;
    const void* Mr = Rb;
    if (opR != bR) {
      if ((r = poetx::launch_superblocks(Rb, nbR, bR, opR, SB, s)) != hipSuccess) return r;
      Mr = SB;
    }
    if ((r = poetx::launch_blockgramapply(gY, Mr, Z, gZ, partR, N, m, opR, plan.sR.nsplit, &ns,
                                          gz_tiled, s)) != hipSuccess)
      return r;
    if ((r = sg.end(0)) != hipSuccess) return r;
    if ((r = sg.begin(1)) != hipSuccess) return r;
    if ((r = poetx::launch_split_reduce(partR, ns, nbR, bR, lastR, GR, gt, s, gram_scale,
                                        plan.subR)) != hipSuccess)
      return r;
    return sg.end(1);
  };
  if (z_saved) {
    POETX_TRY(scale_r());
    if (fuse_r) {
      POETX_TRY(fused_r(z_saved));
    } else {
      POETX_TRY(grad_r());
      POETX_TRY(gram_r(z_saved));
    }
  } else {
    // POET-Xmem: U = X P^T into the g_U buffer and Z = U W0^T into the g_Z
    // buffer (both overwritten later), the R gram on Z, then g_Z over Z
    // (U, read only by the dense kernel, tiled as in the forward)
    const bool u_tiled = dense_direct(t, N, m, n, n, n, m) && apply_tiles(t, N, n, bP);
    POETX_TRY(sg.begin(7));
    POETX_TRY(block_apply(t, X, P_act, gU, N, n, bP, true, s, SB, u_tiled));
    POETX_TRY(dense_forward(t, d, gU, W0, Wq, gZ, nullptr, nullptr, u_tiled, s));
    POETX_TRY(sg.end(7));
    POETX_TRY(scale_r());
    if (fuse_r) {
      POETX_TRY(fused_r(gZ));
    } else {
      POETX_TRY(gram_r(gZ));
      POETX_TRY(grad_r());
    }
  }

  // B3: g_U = g_Z W0   (B(n, k) = W0[k][n])
  POETX_TRY(sg.begin(2));
  POETX_TRY(dense_backward(t, d, gZ, W0, Wq, gU, gz_tiled, s));
  POETX_TRY(sg.end(2));

  if (const int opP = one_pass_size(n, bP)) {
    // B4 and B5 in one pass over g_U (stage 4), then the gram's reduction
    // (stage 3)
    int ns = 0;
    POETX_TRY(sg.begin(4));
    const void* Mp = P_act;
    if (opP != bP) {
      POETX_TRY(poetx::launch_superblocks(P_act, nbP, bP, opP, SB, s));
      Mp = SB;
    }
    POETX_TRY(poetx::launch_blockgramapply(gU, Mp, X, gX, partP, N, n, opP, plan.sP.nsplit, &ns,
                                           false, s));
    POETX_TRY(sg.end(4));
    POETX_TRY(sg.begin(3));
    POETX_TRY(poetx::launch_split_reduce(partP, ns, nbP, bP, lastP, GP, gt, s, nullptr, plan.subP));
    POETX_TRY(sg.end(3));
  } else {
    // B4: G_P[j] = g_U[:, j]^T X[:, j]
    POETX_TRY(sg.begin(3));
    POETX_TRY(block_gram(t, gU, X, partP, N, n, bP, plan.sP, s));
    POETX_TRY(poetx::launch_split_reduce(partP, plan.sP.nsplit, nbP, bP, lastP, GP, gt, s, nullptr,
                                         plan.subP));
    POETX_TRY(sg.end(3));

    // B5: g_X = g_U blockdiag(P)
    POETX_TRY(sg.begin(4));
    POETX_TRY(block_apply(t, gU, P_act, gX, N, n, bP, false, s, SB));
    POETX_TRY(sg.end(4));
  }

  // stage 9 (permutations only): g_x[:, perm_in[j]] = g_X[:, j]
  if (perm) {
    POETX_TRY(sg.begin(9));
    POETX_TRY(poetx::launch_invert_permutation(d->perm_in, (int)n, inv, s));
    POETX_TRY(poetx::launch_gather_columns(t, gX, n, nullptr, N, N, (int)n, inv, g_x, n, s));
    POETX_TRY(sg.end(9));
  }

  // B6: VJP of the orthogonal map for R and for P (one set of launches when
  // b_in == b_out and both sets fit one grid; stage 6 is then empty)
  const bool merged = bR == bP && nbR + nbP <= kMaxBatch;
  if (neumann(d)) {
    // R_f32 / P_f32 hold the skew blocks Q; the partial-gram, T and M
    // buffers are free once the grams are reduced
    if (cnp_bf16) {
      const CnpVjpBf16Set cR{GR, R_f32, partR, TR, MR, g_theta_R, m};
      const CnpVjpBf16Set cP{GP, P_f32, partP, TP, MP, g_theta_P, n};
      POETX_TRY(sg.begin(5));
      POETX_TRY(cnp_vjp_bf16(cR, merged ? &cP : nullptr, bR, s));
      POETX_TRY(sg.end(5));
      POETX_TRY(sg.begin(6));
      if (!merged) POETX_TRY(cnp_vjp_bf16(cP, nullptr, bP, s));
      POETX_TRY(sg.end(6));
    } else {
      const CnpVjpSet cR{GR, R_f32, partR, TR, MR, g_theta_R, m};
      const CnpVjpSet cP{GP, P_f32, partP, TP, MP, g_theta_P, n};
      POETX_TRY(sg.begin(5));
      POETX_TRY(cnp_vjp(cR, merged ? &cP : nullptr, bR, s));
      POETX_TRY(sg.end(5));
      POETX_TRY(sg.begin(6));
      if (!merged) POETX_TRY(cnp_vjp(cP, nullptr, bP, s));
      POETX_TRY(sg.end(6));
    }
  } else {
    const VjpSet vR{GR, R_f32, R_act, TR, MR, g_theta_R, m, saved_y(d)};
    const VjpSet vP{GP, P_f32, P_act, TP, MP, g_theta_P, n, false};
    POETX_TRY(sg.begin(5));
    if (merged && bR > 1) {
      POETX_TRY(cayley_vjp(t, vR, &vP, bR, s));
    } else if (bR > 1) {
      POETX_TRY(cayley_vjp(t, vR, nullptr, bR, s));
    }
    POETX_TRY(sg.end(5));
    POETX_TRY(sg.begin(6));
    if (!merged && bP > 1) POETX_TRY(cayley_vjp(t, vP, nullptr, bP, s));
    POETX_TRY(sg.end(6));
  }
#undef POETX_TRY
  return POETX_OK;
}

int poetx_event_create(void** ev) {
  if (!ev) return POETX_ERR_NULL;
  hipEvent_t e;
  // timing only: recording it skips the system-scope release (a write-back of
  // the caches) that a default event performs between two kernels
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return POETX_ERR_HIP;
  *ev = e;
  return POETX_OK;
}

int poetx_event_destroy(void* ev) {
  if (!ev) return POETX_ERR_NULL;
  return hip_status(hipEventDestroy(static_cast<hipEvent_t>(ev)));
}

int poetx_event_record(void* ev, void* stream) {
  if (!ev) return POETX_ERR_NULL;
  return hip_status(hipEventRecord(static_cast<hipEvent_t>(ev), static_cast<hipStream_t>(stream)));
}

int poetx_event_synchronize(void* ev) {
  if (!ev) return POETX_ERR_NULL;
  return hip_status(hipEventSynchronize(static_cast<hipEvent_t>(ev)));
}

int poetx_event_elapsed_ms(void* a, void* b, float* ms) {
  if (!a || !b || !ms) return POETX_ERR_NULL;
  return hip_status(hipEventElapsedTime(ms, static_cast<hipEvent_t>(a), static_cast<hipEvent_t>(b)));
}

}  // extern "C"
