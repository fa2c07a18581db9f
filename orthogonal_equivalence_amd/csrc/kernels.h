// Internal launcher interface between the C ABI layer (api.cpp) and the HIP
// kernels. Host code only; no torch types anywhere.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace poetx {

enum class DType : int { F32 = 0, BF16 = 1 };

// Batched, split-K GEMM on MFMA:
//   C[s][bt](m, n) = alpha * sum_{k in split s} A[bt](m, k) * B[bt](n, k)
//                    + beta * D[bt](m, n)          (D optional)
// with A(m, k) = A[m*lda + k] when a_kmajor, else A[k*lda + m];
//      B(n, k) = B[n*ldb + k] when b_kmajor, else B[k*ldb + n];
//      C(m, n) = C[m*ldc + n], D(m, n) = D[m*ldd + n].
// Every batch uses extents (M, N, K) except the last, which uses
// (M_last, N_last, K_last) (a ragged, identity-padded last block).
struct GemmParams {
  const void* A = nullptr;
  const void* B = nullptr;
  void* C = nullptr;
  const void* D = nullptr;
  int64_t lda = 0, ldb = 0, ldc = 0, ldd = 0;
  int64_t sA = 0, sB = 0, sC = 0, sD = 0;  // batch strides (elements)
  int M = 0, N = 0, K = 0;
  int M_last = 0, N_last = 0, K_last = 0;
  int batch = 1;
  int ksplit = 1;       // grid.z
  int kchunk = 0;       // K elements per split (multiple of the K tile)
  int64_t sC_split = 0; // output stride between splits (elements)
  float alpha = 1.0f, beta = 0.0f;
  bool d_trans = false;  // D(m, n) = D[n*ldd + m] instead of D[m*ldd + n]
  // Optional second segment: batches >= batch_split use A2/B2/C2/D2 (indexed
  // from batch_split), so two block sets of equal shape share one launch.
  int batch_split = 1 << 30;
  const void* A2 = nullptr;
  const void* B2 = nullptr;
  void* C2 = nullptr;
  const void* D2 = nullptr;
  // Optional bf16 copies of C (and C2) at the same element offsets; only the
  // square float32 kernel (bmm32) writes them, so launch_gemm refuses them
  // for any other path.
  void* C_act = nullptr;
  void* C2_act = nullptr;
};

// Device address of the library's fixed scratch array (POETX_NOALLOC_SCRATCH_BYTES)
// on the current device, looked up once per device; no allocation.
hipError_t noalloc_scratch(void** ptr);

// Returns hipSuccess or the launch error.
hipError_t launch_gemm(DType in, DType out, bool a_kmajor, bool b_kmajor,
                       const GemmParams& p, hipStream_t stream);

// Batched square float32 products (M = N = K a multiple of 128, A K-major,
// B N-major, no split) on the LDS-DMA fp32 kernel; launch_gemm takes this
// path by itself when the shape allows it.
bool bmm32_supported(const GemmParams& p, bool a_kmajor, bool b_kmajor);
hipError_t launch_bmm32(const GemmParams& p, hipStream_t stream);

// K tile of the GEMM configurations for `in` (split-K chunks are multiples
// of it) and the M/N tile chosen for an M x N problem.
int gemm_k_tile(DType in);
int gemm_tile_m(DType in, int M, int N);

// ---- tiled activation layout ----
// A bf16 matrix of R rows (R % 256 == 0) and row length K (K % 32 == 0) in
// the tiled layout holds element (r, k) at
//   ((r / 256) (K / 32) + k / 32) 8192 + (r % 256) 32 + k % 32:
// each 256 x 32 piece is one contiguous 16 KB block, the blocks of a 256-row
// panel in k order (so the panel starts at element 256 K (r / 256), as in the
// row-major layout). The streaming applies can write their output this way
// and the dense kernel can read its A operand this way.
constexpr int kTileRows = 256, kTileCols = 32;
__host__ __device__ inline int64_t tiled_offset(int64_t r, int64_t k, int64_t K) {
  // (r, k >= 0: shifts and masks)
  return (((r >> 8) * (K >> 5) + (k >> 5)) << 13) + ((r & 255) << 5) + (k & 31);
}
static_assert(kTileRows == 256 && kTileCols == 32, "tiled_offset's shifts");

// ---- dense bf16 GEMM with direct-to-LDS loads (the W0 products) ----
// C[M][N] = A[M][K] B(n, k), B(n, k) = B[n*ldb + k] (b_kmajor) or
// B[k*ldb + n]; bf16 in and out, float32 accumulation. With a_tiled, A is in
// the tiled layout (M % 256 == 0 and lda == K, else hipErrorInvalidValue);
// with b_tiled, a K-major B is (an N x K matrix: N % 256 == 0, ldb == K).
bool dense_supported(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc);
hipError_t launch_dense(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                        int64_t lda, int64_t ldb, int64_t ldc, bool b_kmajor, bool a_tiled,
                        bool b_tiled, hipStream_t s);
// nbatch products of that shape, product q at A + q sA, B + q sB, C + q sC
// (elements), in one launch.
hipError_t launch_dense_batched(const void* A, const void* B, void* C, int64_t M, int64_t N,
                                int64_t K, int64_t lda, int64_t ldb, int64_t ldc, bool b_kmajor,
                                int64_t nbatch, int64_t sA, int64_t sB, int64_t sC,
                                hipStream_t s);
// The forward's dense product with the R-apply fused into its epilogue
// (256 x 256 R blocks, bf16): C = A B^T (B K-major) and Y = C blockdiag(R)^T
// with C rounded to bf16 before the second product, as the separate R-apply
// would read it. N must be a multiple of 256; R is [N / 256][256][256]. C
// may be NULL: then only Y is written.
bool dense_fused_r_supported(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                             int64_t ldc, int64_t ldy);
hipError_t launch_dense_fused_r(const void* A, const void* B, void* C, int64_t M, int64_t N,
                                int64_t K, int64_t lda, int64_t ldb, int64_t ldc, const void* R,
                                void* Y, int64_t ldy, bool a_tiled, bool b_tiled, hipStream_t s);

// ---- streaming block-diagonal apply (bf16, b = 128 or 256, b | d) ----
// Y[:, blk] = X[:, blk] M_blk^T (transpose) or X[:, blk] M_blk, token-major
// with row stride d.
bool blockapply_supported(DType t, int64_t d, int b);
// Tokens that one workgroup of the streaming kernel covers for this shape.
int64_t blockapply_tokens_per_workgroup(int64_t tokens, int64_t d, int b);
// Super-block size for block size b (0: none): blocks of b = 32 or 64 are
// run through the b = 128 streaming kernels as block-diagonal 128 x 128
// super blocks (exact zeros off the diagonal), when 128 divides d.
int superblock_size(DType t, int64_t d, int b);
// out[s] = blockdiag(blocks[s S/b], ..., blocks[s S/b + S/b - 1]), S x S bf16,
// for the nblocks (a multiple of S/b) b x b bf16 blocks.
hipError_t launch_superblocks(const void* blocks, int64_t nblocks, int b, int S, void* out,
                              hipStream_t s);
// With y_tiled, Y is written in the tiled layout (row length d; tokens % 256
// == 0, else hipErrorInvalidValue).
hipError_t launch_blockapply(const void* X, const void* M, void* Y, int64_t tokens, int64_t d, int b,
                             bool transpose, bool y_tiled, hipStream_t s);

// Gradient apply and gram of the backward in one pass over X (bf16, b = 128
// or 256):
//   Y[:, blk] = X[:, blk] M_blk   and   part[s][blk] = X[t, blk]^T C[t, blk]
// summed over the tokens of split s. *nsplit (<= max_split) receives the
// number of splits written; the splits cover the tokens in order.
bool blockgramapply_supported(DType t, int64_t d, int b);
// The b = 256 case of launch_blockgramapply: one workgroup per block and
// token range holding the whole block and its whole gram.
// With y_tiled, Y is written in the tiled layout (row length d; tokens % 256
// == 0, else hipErrorInvalidValue); C and Y must then be separate buffers.
hipError_t launch_gramapply256(const void* X, const void* M, const void* C, void* Y, float* part,
                               int64_t tokens, int64_t d, int max_split, int* nsplit, bool y_tiled,
                               hipStream_t s);
hipError_t launch_blockgramapply(const void* X, const void* M, const void* C, void* Y, float* part,
                                 int64_t tokens, int64_t d, int b, int max_split, int* nsplit,
                                 bool y_tiled, hipStream_t s);

// ---- streaming token-reduction grams (bf16, b = 128, 256 or 512, b | d) ----
// part[s][blk] = sum over tokens of split s (kchunk tokens each) of
// A[t, blk]^T C[t, blk], float32 b x b; nsplit * kchunk >= tokens.
bool blockgram_supported(DType t, int64_t d, int b);
// Workgroups per block and token split (b = 512: one per 256 x 256 quadrant).
int blockgram_wg_per_block(int b);
hipError_t launch_blockgram(const void* A, const void* C, float* part, int64_t tokens, int64_t d,
                            int b, int nsplit, int kchunk, hipStream_t s);

// ---- Cayley build (exact Cayley map by blocked Gauss-Jordan) ----
// Panel width used for block size b.
int cayley_panel_width(int b);
// Workspace floats needed by the build for nblocks blocks of size b.
size_t cayley_workspace_floats(int64_t nblocks, int b);
hipError_t launch_cayley_build(const float* theta, int64_t nblocks, int b, int last_valid,
                               float* blocks_f32, void* blocks_act, DType act,
                               float* ws, hipStream_t stream);

// A = diag I + sign Q per block from packed generators (generators of the
// last block's rows/columns >= last_valid taken as zero): I - Q with
// (1, -1), Q itself with (0, 1).
hipError_t launch_expand_skew(const float* theta, int64_t nblocks, int b, int last_valid,
                              float diag, float sign, float* out, hipStream_t stream);

// ---- Cayley-Neumann series (cnp.hip); b % 4 == 0 ----
// RF = I + 2 (E + RF) per block (float32, in place), plus a bf16 copy when
// act_bf16 is not null.
hipError_t launch_cnp_finish(const float* E, float* RF, void* act_bf16, int64_t nblocks, int b,
                             hipStream_t stream);
// C = A - B over n floats (n % 4 == 0, 16-byte aligned pointers).
hipError_t launch_sub(const float* A, const float* B, float* C, int64_t n, hipStream_t stream);
// C (bf16) = A - B with A of type ta and B float32, or C = A when B is NULL
// (a conversion); the difference in float32, rounded once. n % 4 == 0, A and
// C 8-byte aligned, B 16-byte aligned. A second set (A2, B2, C2, n2
// elements, the same rules; n2 = 0 for none) shares the launch.
hipError_t launch_sub_to_bf16(DType ta, const void* A, const float* B, void* C, int64_t n,
                              const void* A2, const float* B2, void* C2, int64_t n2,
                              hipStream_t stream);
// W = S + S^T per b x b block, S = A + B.
hipError_t launch_sym_sum(const float* A, const float* B, float* W, int64_t nblocks, int b,
                          hipStream_t stream);
// The same for bf16 A, B and W (the sums in float32, W rounded once), with
// an optional second set of nblocks2 blocks in the same launch.
hipError_t launch_sym_sum_bf16(const void* A, const void* B, void* W, int64_t nblocks,
                               const void* A2, const void* B2, void* W2, int64_t nblocks2, int b,
                               hipStream_t stream);

// ---- block-mixing permutations (permute.hip) ----
// out[r][j] = in[src][perm[j]] for r < rows, j < d, src = rowmap ? rowmap[r] : r;
// indices outside [0, d) (or a src outside [0, in_rows)) read as zero.
// d, ld_in, ld_out multiples of 16 bytes / element size; out must not overlap in.
hipError_t launch_gather_columns(DType t, const void* in, int64_t ld_in, const int32_t* rowmap,
                                 int64_t in_rows, int64_t rows, int d, const int32_t* perm,
                                 void* out, int64_t ld_out, hipStream_t s);
// inv[perm[i]] = i for in-range entries, -1 elsewhere (two small launches).
hipError_t launch_invert_permutation(const int32_t* perm, int d, int32_t* inv, hipStream_t s);

// ---- INT8 frozen weight (quant.hip) ----
// Per-row symmetric codes: scale[r] = amax / 127, q = clamp(rint(w / scale)),
// float32 correctly rounded divisions; d % 8 == 0.
hipError_t launch_quantize_rows(DType t, const void* W, int64_t rows, int d, int8_t* q,
                                float* scale, hipStream_t s);
// out[r][j] = q[r ldq + j] in the activation type (exact) for r < rows,
// j < cols: a rows x cols slice of the codes (row stride ldq) into a
// contiguous rows x cols matrix; cols and ldq multiples of 8, q 8-byte
// aligned. With out_tiled, out is in the tiled layout (rows % 256 == 0,
// cols % 32 == 0).
hipError_t launch_widen_codes(DType t, const int8_t* q, int64_t rows, int64_t ldq, int64_t cols,
                              void* out, bool out_tiled, hipStream_t s);
// out[k][i][j] = M[k][i][j] * scale[k b + j] (0 past d), activation type.
hipError_t launch_scale_block_columns(DType t, const void* M, const float* scale, int64_t nblocks,
                                      int b, int64_t d, void* out, hipStream_t s);

// ---- backward helpers ----
// G[blk] = sum_s part[s][blk] in split order (float32), stored as `out`;
// entries of the last block at rows or columns >= last_valid are zero. With
// col_scale, column j of block blk is multiplied by col_scale[blk b + j].
hipError_t launch_split_reduce(const float* part, int nsplit, int64_t nblocks, int b,
                               int last_valid, void* G, DType out, hipStream_t stream,
                               const float* col_scale = nullptr, int sub = 1);
// g_theta[blk][idx(i,j)] = sign ((M + c S)[i][j] - (M + c S)[j][i]) (i < j),
// S an optional bf16 addend; zero for entries of the last block at rows or
// columns >= last_valid. A second set of blocks of the same size shares the
// launch.
struct PackSet {
  const float* M;
  const void* S;
  int64_t nblocks;
  int last_valid;
  float* g_theta;
};
hipError_t launch_pack_skew_grad(const PackSet& a, const PackSet* b2, float c, int b, float sign,
                                 hipStream_t stream);

}  // namespace poetx
