/*
 * poetx.h - C ABI of libpoetx, the POET-X linear layer y = R W0 P x on
 * MI355X (gfx950).
 *
 * Method sources (every page carries the title "POET-X: Memory-efficient LLM
 * Training by Scaling Orthogonal Transformation"; the technical text is the
 * German summary on gist.science, "Technische Zusammenfassung"):
 *   - weight reparameterisation W = R W0 P with trainable orthogonal R, P and
 *     a frozen W0: section 1 (Problemstellung);
 *   - input-centric evaluation (transform the activations, never rebuild W):
 *     section 2 (Methodik), input-centric formulation item;
 *   - block-diagonal R and P whose blocks are multiplied as independent
 *     matrices in a batch: section 2, batch-parallel block-diagonal item;
 *   - skew-symmetric generators Q = -Q^T stored as their upper triangle only:
 *     section 2, Cayley-Neumann parameterisation item.
 * The orthogonal map is the exact Cayley map R = (I + Q)(I - Q)^-1. The
 * backward (to the activations and to the generators) is the chain rule of
 * that forward; the pages do not spell it out.
 *
 * Conventions shared by every call
 *   - Every tensor pointer is a DEVICE pointer owned by the caller. The
 *     library never allocates or frees memory and never synchronises: calls
 *     validate their arguments on the host, enqueue kernels on `stream` (a
 *     hipStream_t; NULL is the default stream) and return.
 *   - Tensors are dense and row-major. Activations are token-major:
 *     x [tokens, d_in], y and z [tokens, d_out]. W0 is [d_out, d_in].
 *   - A block size b splits d features into nb = ceil(d / b) contiguous
 *     blocks starting at feature 0. If b does not divide d the last block
 *     holds r = d - (nb - 1) b features and is identity-padded: its generator
 *     entries in rows or columns >= r are ignored (treated as zero) and their
 *     gradients are written as zero.
 *   - Generators theta are float32 [nb, b(b-1)/2]: the strict upper triangle
 *     of each b x b skew block, packed row by row, so entry (i, j), i < j, is
 *     at i(2b - i - 1)/2 + (j - i - 1). Q[i][j] = theta, Q[j][i] = -theta.
 *   - Orthogonal blocks are [nb, b, b] row-major. R block k maps output
 *     features [k b, k b + b); P block j maps input features [j b, j b + b).
 *     Token-major, the layer is Y = X blockdiag(P)^T W0^T blockdiag(R)^T.
 *   - `act` selects the storage type (poetx_dtype) of x, W0, y, z, g_y, g_x
 *     and of the *_act copies of the blocks. theta, the float32 blocks and
 *     g_theta are float32 in both modes. All accumulation is float32; bf16
 *     results are rounded to nearest even.
 *   - Alignment: every tensor pointer is 16-byte aligned; d_in, d_out and b
 *     are multiples of 8 (bf16) or 4 (float32).
 *   - Outputs are overwritten (not accumulated into) and must not overlap any
 *     input. Calls that share a workspace must not run concurrently.
 *   - Errors: argument faults are detected on the host before any launch and
 *     returned as a status; nothing is enqueued then. A failed launch returns
 *     POETX_ERR_HIP. Non-finite inputs are not trapped (NaN in, NaN out).
 *     Nothing throws across this interface and the library keeps no state
 *     between calls, except the fixed scratch area of
 *     poetx_linear_fwd_noalloc.
 */
#ifndef POETX_H
#define POETX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define POETX_ABI_VERSION 7

typedef enum poetx_status {
  POETX_OK = 0,
  POETX_ERR_NULL = 1,      /* a required pointer is NULL */
  POETX_ERR_SHAPE = 2,     /* a size is out of range or inconsistent */
  POETX_ERR_DTYPE = 3,     /* unknown poetx_dtype */
  POETX_ERR_ALIGN = 4,     /* a pointer or size breaks the alignment rule */
  POETX_ERR_WORKSPACE = 5, /* workspace NULL or smaller than required */
  POETX_ERR_HIP = 6,       /* the HIP runtime reported an error */
  POETX_ERR_ALIAS = 7      /* an output overlaps an input */
} poetx_status;

typedef enum poetx_dtype { POETX_F32 = 0, POETX_BF16 = 1 } poetx_dtype;

/* poetx_linear_desc.flags */
/* Recompute Z in the backward instead of keeping it (POET-Xmem: section 2
 * Methodik, gradient-checkpointing item; some forward intermediates are not
 * stored but recomputed in the backward). With this flag the
 * forward takes z_save == NULL and keeps Z in its workspace only, and the
 * backward takes z_saved == NULL and recomputes U = X P^T and Z = U W0^T in
 * its own workspace (one extra dense product). Results are those of the
 * stored-Z path. */
#define POETX_RECOMPUTE_Z 1
/* The blocks were built by the truncated Cayley-Neumann series
 * (poetx_build_cnp) rather than the exact Cayley map: the backward then takes
 * the skew blocks Q in place of the float32 orthogonal blocks and applies the
 * series' VJP (section 2 Methodik, Cayley-Neumann parameterisation item). */
#define POETX_CAYLEY_NEUMANN 2
/* Keep the layer's output Y for the backward in place of Z. R is orthogonal,
 * so per block Z = Y R and the R gram g_Y^T Z equals (g_Y^T Y) R: the
 * backward forms g_Y^T Y from y and takes the factor R into the first
 * product of the Cayley VJP, M = 1/2 (R^T + I) (g_Y^T Y)(I + R), which costs
 * what M = 1/2 (R^T + I) G (R^T + I) costs. A caller whose next operation
 * keeps y anyway (an activation function, attention) then holds no
 * [tokens, d_out] tensor for this layer. The forward takes z_save == NULL;
 * with 256 x 256 bf16 R blocks (R-apply inside the dense product) it writes
 * no Z at all, otherwise Z lives in its workspace. The backward takes the
 * forward's y as z_saved. Agrees with the stored-Z path up to rounding: the
 * identity is exact for orthogonal blocks, and the act-type blocks of bf16
 * mode are orthogonal to about 2^-8. With an INT8 weight the R gram then
 * needs no column scaling (Y already carries the scales). Not together with
 * POETX_RECOMPUTE_Z, with POETX_CAYLEY_NEUMANN (the truncated series is not
 * exactly orthogonal) or with permutations (y is in permuted column order):
 * POETX_ERR_SHAPE. */
#define POETX_SAVED_Y 4

/* Shape of one POET-X linear layer. */
typedef struct poetx_linear_desc {
  int64_t tokens; /* N >= 1: rows of x, y, z, g_y, g_x */
  int64_t d_in;   /* n: input features (columns of W0) */
  int64_t d_out;  /* m: output features (rows of W0) */
  int32_t b_in;   /* block size of P, 1 <= b_in <= d_in rounded up to a block */
  int32_t b_out;  /* block size of R */
  int32_t act;    /* poetx_dtype of the activations, W0 and the *_act blocks */
  int32_t n_events; /* number of entries in `events` (0 = no stage timing) */
  int32_t flags;    /* 0 or POETX_RECOMPUTE_Z | POETX_CAYLEY_NEUMANN | POETX_SAVED_Y */
  int32_t reserved; /* must be 0 */
  /* Optional stage timing: an array of hipEvent_t created by the caller (for
   * example with poetx_event_create). When n_events >= 2 s + 2, the call
   * records events[2 s] on `stream` before its stage s and events[2 s + 1]
   * after it. Forward stages: 0 P-apply, 1 dense W0 GEMM, 2 R-apply.
   * Backward stages: 0 grad through R, 1 R gram (+ reduction), 2 dense W0
   * GEMM, 3 P gram (+ reduction), 4 grad to x, 5 Cayley VJP of R,
   * 6 Cayley VJP of P, 7 recompute of Z (POETX_RECOMPUTE_Z only; it runs
   * first, and stage 1 then runs before stage 0). Where the gradient apply
   * and the gram of a side share one pass (bf16 with b = 128 or 256, or
   * b = 32 / 64 when 128 divides the side's width), stage 0 (R side) or 4
   * (P side) holds that pass and stage 1 or 3 the gram's reduction alone,
   * run after it. With permutations, forward
   * stage 3 gathers x and stage 4 scatters y; backward stage 8 gathers g_y
   * and x and stage 9 scatters g_x. With an INT8 weight, forward stage 5 and
   * backward stage 10 scale R's block columns (the codes are widened chunk
   * by chunk inside the dense stages: forward 1, backward 2 and 7). A NULL
   * entry is skipped, so a caller can time one stage alone (each record adds
   * a few microseconds between kernels). May be NULL when n_events is 0. */
  void* const* events;
  /* Optional block-mixing permutations (section 2 Methodik, permutation
   * item): index maps perm_in [d_in] and perm_out [d_out], int32 device
   * arrays (4-byte aligned), both or neither (NULL: no permutation). With
   * them the layer is
   *   y = Pi_out^T blockdiag(R) Pi_out W0 Pi_in^T blockdiag(P) Pi_in x,
   * (Pi v)_i = v[perm[i]], and the W0 argument of the forward and backward
   * is the folded weight W0' = Pi_out W0 Pi_in^T (poetx_fold_weight), so
   * only the two outer permutations run per call: x's columns are gathered by
   * perm_in, y's scattered by perm_out (the backward mirrors this). Each map
   * must be a permutation of 0..d-1; an entry outside that range reads as
   * zero (never an out-of-bounds access), a repeated entry leaves the result
   * unspecified. */
  const int32_t* perm_in;
  const int32_t* perm_out;
  /* Optional INT8 frozen weight (section 2 Methodik, quantised-support item,
   * POET-XQ). NULL: W0 is in the act type. Otherwise W0 holds int8 codes
   * q [d_out, d_in] and w_scale [d_out] float32 row scales
   * (poetx_quantize_weight), the layer's weight being diag(w_scale) q
   * exactly; d_in must be a multiple of 8. The codes are widened to the act
   * type without rounding, a chunk of weight rows (forward) or columns
   * (backward) at a time, each enough for about one round of the dense
   * product's output tiles, into the workspace; so the workspace holds only a
   * fraction of the weight in the act type. The scales enter through R: the forward
   * computes Z_q = U q^T and Y = Z_q (blockdiag(R) diag(s))^T and keeps Z_q as
   * z_save; the backward uses g_Z' = g_Y blockdiag(R) diag(s),
   * g_U = g_Z' q and G_R = (g_Y^T Z_q) diag(s). */
  const float* w_scale;
} poetx_linear_desc;

/* Returns POETX_ABI_VERSION. */
int poetx_abi_version(void);

/* Static text for a status code ("unknown status" for other values). */
const char* poetx_status_string(int status);

/* ceil(d / b); 0 if d < 1 or b < 1. */
int64_t poetx_num_blocks(int64_t d, int32_t b);

/* Number of float32 generators for d features in blocks of b:
 * ceil(d / b) * b (b - 1) / 2; 0 if d < 1 or b < 1. */
int64_t poetx_theta_count(int64_t d, int32_t b);

/* Workspace bytes poetx_build_orthogonal needs for d features, block size b
 * (0 for invalid sizes). */
size_t poetx_build_workspace_size(int64_t d, int32_t b);

/*
 * poetx_build_orthogonal - packed skew generators to orthogonal blocks.
 * (Cayley-Neumann parameterisation item of section 2: skew generators stored
 * as the upper triangle; exact Cayley map.)
 *
 *   theta       [nb, b(b-1)/2] float32, nb = ceil(d / b). May be NULL only if
 *               b == 1 (no generators).
 *   d, b        features covered and block size; 1 <= b <= 4096, d >= 1.
 *               Several block sets with the same b (for example R and P of
 *               a layer, or every layer of a model) may be built in one call
 *               by storing their generators back to back and passing the
 *               summed feature count, provided b divides each set's d.
 *   blocks_f32  out [nb, b, b] float32: R_k = (I + Q_k)(I - Q_k)^-1, computed
 *               as 2 (I - Q_k)^-1 - I by unpivoted blocked Gauss-Jordan
 *               elimination (I - Q has symmetric part I, so no pivot is ever
 *               needed); from 48 blocks of 512, as 2 x 2 pieces of 256 joined
 *               through the Schur complement of the leading piece (whose
 *               symmetric part is positive definite too). The rounding of
 *               the float32 result depends on which of these forms runs, so
 *               a block built alone and in a large set may differ in the last
 *               bits.
 *   blocks_act  out [nb, b, b] copy in `act` type (bf16: round to nearest
 *               even). Required when act is POETX_BF16; ignored (may be NULL)
 *               when act is POETX_F32.
 *   ws          workspace of at least poetx_build_workspace_size(d, b) bytes.
 */
int poetx_build_orthogonal(const float* theta, int64_t d, int32_t b,
                           float* blocks_f32, void* blocks_act, int32_t act,
                           void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes poetx_build_cnp needs for d features, block size b (0 for
 * invalid sizes, including b not a multiple of 4). */
size_t poetx_build_cnp_workspace_size(int64_t d, int32_t b);

/*
 * poetx_build_cnp - packed skew generators to blocks by the truncated
 * Cayley-Neumann series (section 2 Methodik, Cayley-Neumann parameterisation
 * item: the Cayley map approximated by a Neumann series whose higher terms
 * are Q^2, Q^3, Q^4). The series truncates (I - Q)^-1 inside
 * R = 2 (I - Q)^-1 - I:
 *   R_k = I + 2 (Q_k + Q_k^2 + Q_k^3 + Q_k^4),
 * orthogonal only up to O(|Q|^6) and divergent from the exact map for
 * |Q| >= 1. Products in float32 on MFMA.
 *
 *   theta, d, act, blocks_act, ws  as for poetx_build_orthogonal, with
 *               ws of poetx_build_cnp_workspace_size(d, b) bytes.
 *   b           block size, 4 <= b <= 4096, b % 4 == 0 (else POETX_ERR_ALIGN).
 *   q_f32       out [nb, b, b] float32: the skew blocks Q_k (generators of a
 *               padded last block's rows/columns past d are zero). Pass them
 *               as R_f32 / P_f32 to poetx_linear_bwd with POETX_CAYLEY_NEUMANN.
 *   blocks_f32  out [nb, b, b] float32: R_k.
 * Errors as poetx_build_orthogonal; q_f32 must overlap no other argument.
 */
int poetx_build_cnp(const float* theta, int64_t d, int32_t b, float* q_f32, float* blocks_f32,
                    void* blocks_act, int32_t act, void* ws, size_t ws_bytes, void* stream);

/*
 * poetx_fold_weight - the two inner permutations of the forward folded into
 * the frozen weight once (section 2 Methodik, permutation item, reduction):
 *   W0_folded[i][j] = W0[perm_out[i]][perm_in[j]]   (W0' = Pi_out W0 Pi_in^T)
 *
 *   W0, W0_folded  [d_out, d_in] in `act` type, 16-byte aligned, no overlap
 *   perm_out       [d_out] int32, perm_in [d_in] int32 (device, 4-byte aligned);
 *                  out-of-range entries read as zero
 * Errors: POETX_ERR_DTYPE, POETX_ERR_SHAPE (d < 1), POETX_ERR_NULL,
 * POETX_ERR_ALIGN (d_in not a multiple of 8 for bf16 / 4 for float32, or a
 * pointer), POETX_ERR_ALIAS, POETX_ERR_HIP.
 */
int poetx_fold_weight(const void* W0, int64_t d_out, int64_t d_in, const int32_t* perm_out,
                      const int32_t* perm_in, int32_t act, void* W0_folded, void* stream);

/*
 * poetx_quantize_weight - symmetric per-row INT8 codes of a weight (the
 * scheme is not given on the pages; this one is):
 *   scale[i] = amax_j |W0[i][j]| / 127,
 *   q[i][j]  = clamp(rint(W0[i][j] / scale[i]), -127, 127)
 * with both divisions correctly rounded in float32 and rint rounding half to
 * even; an all-zero row gets scale 0 and codes 0. Weights must be finite.
 *
 *   W0     [d_out, d_in] in `act` type, 16-byte aligned
 *   q      out [d_out, d_in] int8, 16-byte aligned
 *   scale  out [d_out] float32, 4-byte aligned
 * Errors: POETX_ERR_DTYPE, POETX_ERR_SHAPE (d < 1), POETX_ERR_NULL,
 * POETX_ERR_ALIGN (d_in not a multiple of 8, or a pointer), POETX_ERR_ALIAS,
 * POETX_ERR_HIP. Folding permutations first and then quantising gives the
 * same codes as quantising first and folding (the row maxima are unchanged).
 */
int poetx_quantize_weight(const void* W0, int64_t d_out, int64_t d_in, int32_t act, int8_t* q,
                          float* scale, void* stream);

/* Workspace bytes for poetx_linear_fwd / poetx_linear_bwd (0 if the
 * descriptor is invalid). With POETX_RECOMPUTE_Z the forward's includes Z,
 * and with POETX_SAVED_Y too unless the R-apply runs inside the dense
 * product. */
size_t poetx_fwd_workspace_size(const poetx_linear_desc* desc);
size_t poetx_bwd_workspace_size(const poetx_linear_desc* desc);

/*
 * poetx_linear_fwd - forward of the layer, input-centric (section 2,
 * input-centric formulation; blocks applied batch-parallel):
 *   U = X blockdiag(P)^T, Z = U W0^T, Y = Z blockdiag(R)^T.
 *
 *   x      [tokens, d_in]  act
 *   W0     [d_out, d_in]   act (frozen base weight), or int8 codes when
 *          desc->w_scale is set
 *   R_act  [nb_out, b_out, b_out] act, from poetx_build_orthogonal
 *   P_act  [nb_in,  b_in,  b_in ] act
 *   y      out [tokens, d_out] act
 *   z_save out [tokens, d_out] act: Z, kept for the backward; NULL (and
 *          only NULL) when desc->flags has POETX_RECOMPUTE_Z or
 *          POETX_SAVED_Y
 *   ws     workspace of poetx_fwd_workspace_size(desc) bytes
 */
int poetx_linear_fwd(const poetx_linear_desc* desc, const void* x, const void* W0,
                     const void* R_act, const void* P_act, void* y, void* z_save,
                     void* ws, size_t ws_bytes, void* stream);

/* Bytes of the library's fixed device scratch area used by
 * poetx_linear_fwd_noalloc (one copy per GPU, held until the process ends). */
#define POETX_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * poetx_linear_fwd_noalloc - poetx_linear_fwd for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and results, with the
 * forward's workspace taken from a scratch array inside the library instead
 * of a caller-provided buffer. The call itself allocates and frees nothing.
 *
 *   desc, x, W0, R_act, P_act, y, z_save, stream  as for poetx_linear_fwd.
 *
 * Limit: poetx_fwd_workspace_size(desc) must not exceed
 * POETX_NOALLOC_SCRATCH_BYTES (64 MiB: for example 8192 tokens x 4096 input
 * features in bf16); a larger workspace returns POETX_ERR_WORKSPACE before
 * anything is enqueued. Other argument faults are reported as by
 * poetx_linear_fwd, also before anything is enqueued; POETX_ERR_HIP if the
 * scratch area's device address cannot be obtained (it is looked up once per
 * device, on that device's first call).
 * Every call on one GPU uses the same scratch area, which keeps the last
 * call's contents (nothing in it needs to start at zero): calls that overlap
 * on one GPU (other streams, other host threads) race and must be
 * serialised by the caller.
 */
int poetx_linear_fwd_noalloc(const poetx_linear_desc* desc, const void* x, const void* W0,
                             const void* R_act, const void* P_act, void* y, void* z_save,
                             void* stream);

/*
 * poetx_linear_bwd - backward of the layer to the activations and to the
 * generators (chain rule of the forward above; W0 is frozen, so no gradient
 * for it is formed):
 *   g_Z = g_Y blockdiag(R)          G_R[k] = g_Y[:, k]^T Z[:, k]
 *   g_U = g_Z W0                    G_P[j] = g_U[:, j]^T X[:, j]
 *   g_X = g_U blockdiag(P)
 *   Cayley VJP per block: M = 1/2 (R^T + I) G (R^T + I),
 *   g_theta(i, j) = M[i][j] - M[j][i] for i < j
 *   (bf16 mode: G and T = G R^T + G are rounded to bf16 for the two VJP
 *   products, which accumulate in float32).
 *   With POETX_CAYLEY_NEUMANN, the series' VJP instead:
 *   D = 2 sum_{k=1..4} sum_{i+j=k-1} (Q^T)^i G (Q^T)^j,
 *   g_theta(i, j) = D[i][j] - D[j][i], in float32; in bf16 mode with
 *   b_in and b_out multiples of 8, its products take bf16 operands (G, Q
 *   and the intermediate products rounded to bf16) and accumulate in
 *   float32.
 * The token reductions are split over workgroups and summed in a fixed
 * order, so results are bitwise reproducible.
 *
 *   g_y        [tokens, d_out] act
 *   x          [tokens, d_in]  act
 *   W0         [d_out, d_in]   act
 *   R_f32      [nb_out, b_out, b_out] float32, P_f32 [nb_in, b_in, b_in] float32:
 *              the orthogonal blocks, or with POETX_CAYLEY_NEUMANN the skew
 *              blocks q_f32 of poetx_build_cnp
 *   R_act, P_act  the act copies of the orthogonal blocks
 *   z_saved    [tokens, d_out] act, z_save of the matching forward; with
 *              POETX_SAVED_Y its y instead; NULL (and only NULL) when
 *              desc->flags has POETX_RECOMPUTE_Z
 *   g_x        out [tokens, d_in] act
 *   g_theta_R  out [nb_out, b_out(b_out-1)/2] float32
 *   g_theta_P  out [nb_in,  b_in(b_in-1)/2]   float32
 *   ws         workspace of poetx_bwd_workspace_size(desc) bytes
 */
int poetx_linear_bwd(const poetx_linear_desc* desc, const void* g_y, const void* x,
                     const void* W0, const float* R_f32, const float* P_f32,
                     const void* R_act, const void* P_act, const void* z_saved,
                     void* g_x, float* g_theta_R, float* g_theta_P,
                     void* ws, size_t ws_bytes, void* stream);

/* Thin hipEvent helpers so a caller without HIP headers can time stages.
 * Each returns a poetx_status. The events are for timing only: they are
 * created with hipEventDisableSystemFence, so recording one between two
 * kernels does not write back the caches, and synchronizing on one does not
 * make the timed work's results visible to the host (synchronize the stream
 * or device for that). */
int poetx_event_create(void** event);
int poetx_event_destroy(void* event);
int poetx_event_record(void* event, void* stream);
int poetx_event_synchronize(void* event);
int poetx_event_elapsed_ms(void* start, void* stop, float* ms);

#ifdef __cplusplus
}
#endif

#endif /* POETX_H */
