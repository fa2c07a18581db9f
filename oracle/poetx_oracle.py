"""Float64 CPU oracle of the POET-X linear layer y = R W0 P x.

TEST INFRASTRUCTURE. Only tests, the smoke check and the benchmark's CPU
baseline may import or run this module; the library and its Python binding
never do. It shares no code with the HIP path.

Sources (all pages carry the title "POET-X: Memory-efficient LLM Training by
Scaling Orthogonal Transformation"; the technical text is the German summary
on gist.science, "Technische Zusammenfassung"):
  [OET]   §1 Problemstellung: a weight is reparameterised as W = R W0 P, with
          R and P trainable orthogonal matrices; the ICML and arXiv abstracts
          add that the transform preserves the singular spectrum.
  [IC]    §2 Methodik, input-centric formulation: instead of rebuilding the
          weight, the transform is applied to the activations, one operation
          after another.
  [BD]    §2 Methodik, batch-parallel block-diagonal matrices: R and P are
          block-diagonal and their blocks are multiplied as independent
          matrices.
  [SKEW]  §2 Methodik, Cayley-Neumann parameterisation: orthogonality comes
          from a skew-symmetric Q (Q = -Q^T) of which only the upper triangle
          is stored.
  [CNP]   same item: the Cayley map is approximated by a truncated Neumann
          series whose higher-order terms are Q^2, Q^3 and Q^4.
  [PERM]  §2 Methodik, permutation item: permutation matrices mix the blocks
          of the orthogonal matrices; they are applied as index maps
          (bijections) on the data, and two of the four permutations of the
          forward pass are folded into the weight in advance.
  [XQ]    §2 Methodik, quantised-support item (POET-XQ): since the transform
          acts on the activations and no high-precision copy of the weight
          has to be kept, the frozen weight may be a quantised (e.g. INT8)
          model.

Readings taken where the pages are silent:
  * the orthogonal map is the exact Cayley map R = (I + Q)(I - Q)^-1 (the
    pages name a truncated-series approximation of it without printing it);
    the sign convention is the one whose series expansion of (I - Q)^-1 has
    only positive powers of Q, matching the pages' list of powers Q..Q^4;
  * Q is built as U - U^T from the strict upper triangle U, no 1/2 factor,
    packed row-major: idx(i, j) = i(2b - i - 1)/2 + (j - i - 1) for i < j;
  * R acts on the d_out outputs, P on the d_in inputs; blocks are contiguous
    and start at feature 0; no permutation;
  * if b does not divide d, the last block is identity-padded: the generator
    entries of rows/columns past the end are treated as zero, so the block is
    diag(Cayley(Q_r), I) and only its leading r x r part acts;
  * backward outputs are g_x, g_theta_R, g_theta_P (W0 is frozen, no g_W0);
  * the Cayley-Neumann variant (selected explicitly; the exact map is the
    default) truncates (I - Q)^-1 = I + Q + Q^2 + ... after Q^4 inside
    R = 2 (I - Q)^-1 - I, so R = I + 2 (Q + Q^2 + Q^3 + Q^4): only the
    powers the pages list occur. (Truncating inside (I + Q)(I - Q)^-1 would
    add a Q^5 term; that reading is not taken.)
  * with block-mixing permutations (optional; none by default) the
    orthogonal factors are R = Pi_R^T blockdiag(R_k) Pi_R and
    P = Pi_P^T blockdiag(P_j) Pi_P, where (Pi v)_i = v[pi(i)] for an index
    map pi; these are the four permutations of the forward, and the inner
    two fold into W0' = Pi_R W0 Pi_P^T, W0'[i][j] = W0[pi_R(i)][pi_P(j)];
  * INT8 weights (optional) are symmetric with one float32 scale per output
    row: s_i = amax_i / 127 and q_ij = clamp(rint(w_ij / s_i), -127, 127),
    both divisions in float32 (round to nearest even), s_i = 0 and q = 0 for
    an all-zero row; the layer then uses W0 = diag(s) q exactly.

Where "parity unpinned": nothing here. Every function is pinned by
tests/test_oracle.py against closed forms (b = 2 rotation, b = 3 Rodrigues
rotation, the b = 2 Cayley-Neumann block and its derivative), invariants
(orthogonality, det, spectrum, the series tail 2 Q^5 (I - Q)^-1 between the
exact and truncated maps), textbook routines (dense scipy block_diag
products), the block-triangular Frechet identity and central finite
differences.

Layouts: activations are token-major, x [N, d_in], y [N, d_out]; W0 is
[d_out, d_in]; theta is [nblocks, b(b-1)/2].
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

__all__ = [
    "packed_upper_index", "skew_from_theta", "theta_from_skew", "cayley",
    "block_ranges", "orthogonal_blocks", "materialise", "forward",
    "backward", "cayley_vjp", "forward_input_centric",
    "backward_input_centric", "LayerOracle", "CNP_ORDER", "cayley_neumann",
    "cayley_neumann_vjp", "orthogonal_blocks_cnp", "permutation_matrix",
    "fold_permutations", "materialise_permuted", "quantize_rows", "dequantize_rows",
]


# ---------------------------------------------------------------- [SKEW]
def packed_upper_index(b: int) -> Tuple[np.ndarray, np.ndarray]:
    """Row/column indices (i < j) of the packed strict upper triangle, in
    storage order: row-major, so position p holds Q[i[p], j[p]] with
    p = i(2b - i - 1)/2 + (j - i - 1). [SKEW]"""
    rows, cols = [], []
    for i in range(b):
        for j in range(i + 1, b):
            rows.append(i)
            cols.append(j)
    return np.asarray(rows, dtype=np.int64), np.asarray(cols, dtype=np.int64)


def skew_from_theta(theta: np.ndarray, b: int, d: int | None = None) -> np.ndarray:
    """Expand packed generators theta [nb, b(b-1)/2] to skew blocks Q [nb, b, b]
    with Q[i, j] = theta, Q[j, i] = -theta for i < j and a zero diagonal.
    [SKEW] If `d` is given and b does not divide it, the entries of the last
    block's rows and columns at or past r = d - (nb-1) b are zeroed
    (identity padding)."""
    theta = np.asarray(theta, dtype=np.float64)
    nb = theta.shape[0]
    iu, ju = packed_upper_index(b)
    Q = np.zeros((nb, b, b), dtype=np.float64)
    Q[:, iu, ju] = theta
    Q[:, ju, iu] = -theta
    if d is not None:
        r = d - (nb - 1) * b
        if r < b:
            Q[-1, r:, :] = 0.0
            Q[-1, :, r:] = 0.0
    return Q


def theta_from_skew(Q: np.ndarray) -> np.ndarray:
    """Pack the strict upper triangle of each block of Q [nb, b, b]. [SKEW]"""
    b = Q.shape[-1]
    iu, ju = packed_upper_index(b)
    return np.ascontiguousarray(Q[:, iu, ju])


# ------------------------------------------------------ exact Cayley map
def cayley(Q: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Exact Cayley map of each skew block: B = (I - Q)^-1 by a LAPACK solve
    (partial pivoting), then R = (I + Q) B. Returns (R, B), each [nb, b, b].
    [SKEW] names the Cayley-based parameterisation; the exact map is this
    build's reading (see the module docstring)."""
    Q = np.asarray(Q, dtype=np.float64)
    b = Q.shape[-1]
    I = np.eye(b)
    B = np.stack([np.linalg.solve(I - q, I) for q in Q]) if len(Q) else np.zeros_like(Q)
    R = np.stack([(I + q) @ bk for q, bk in zip(Q, B)]) if len(Q) else np.zeros_like(Q)
    return R, B


# ----------------------------------------- Cayley-Neumann series [CNP]
CNP_ORDER = 4  # highest power of Q kept: the pages list Q^2, Q^3, Q^4


def cayley_neumann(Q: np.ndarray) -> np.ndarray:
    """Truncated Cayley map of each skew block: (I - Q)^-1 is replaced by its
    Neumann series up to Q^4 in R = 2 (I - Q)^-1 - I, so
    R = I + 2 (Q + Q^2 + Q^3 + Q^4). [CNP] Powers are formed one after the
    other, Q^k = Q^(k-1) Q. Returns R [nb, b, b]; orthogonal only up to
    O(|Q|^6)."""
    Q = np.asarray(Q, dtype=np.float64)
    b = Q.shape[-1]
    I = np.eye(b)
    out = np.empty_like(Q)
    for k, q in enumerate(Q):
        series = np.zeros((b, b))
        power = I
        for _ in range(CNP_ORDER):
            power = power @ q
            series = series + power
        out[k] = I + 2.0 * series
    return out


def cayley_neumann_vjp(Q: np.ndarray, G: np.ndarray) -> np.ndarray:
    """Gradient of the packed generators given G = dL/dR per block, for
    R = I + 2 sum_{k=1..4} Q^k.

    d(Q^k) = sum_{i+j=k-1} Q^i dQ Q^j, so
    dL/dQ = 2 sum_{k=1..4} sum_{i+j=k-1} (Q^T)^i G (Q^T)^j, and, as for the
    exact map, dL/dtheta_(i,j) = D[i, j] - D[j, i] with D = dL/dQ.
    (The chain rule of the series; the pages describe no backward.)"""
    b = Q.shape[-1]
    iu, ju = packed_upper_index(b)
    out = np.empty((Q.shape[0], len(iu)), dtype=np.float64)
    for n in range(Q.shape[0]):
        Qt = Q[n].T
        pw = [np.eye(b)]
        for _ in range(CNP_ORDER - 1):
            pw.append(pw[-1] @ Qt)
        D = np.zeros((b, b))
        for k in range(1, CNP_ORDER + 1):
            for i in range(k):
                D += pw[i] @ G[n] @ pw[k - 1 - i]
        D *= 2.0
        out[n] = D[iu, ju] - D[ju, iu]
    return out


# ------------------------------------------------------- block structure
def block_ranges(d: int, b: int) -> List[Tuple[int, int]]:
    """(start, size) of each contiguous block of features; the last block may
    be shorter when b does not divide d. [BD]"""
    return [(s, min(b, d - s)) for s in range(0, d, b)]


def orthogonal_blocks(theta: np.ndarray, b: int, d: int) -> Tuple[np.ndarray, np.ndarray]:
    """theta [nb, b(b-1)/2] -> (R blocks, B blocks) of a block-diagonal
    orthogonal matrix on d features. [SKEW], [BD]"""
    return cayley(skew_from_theta(theta, b, d))


def orthogonal_blocks_cnp(theta: np.ndarray, b: int, d: int) -> Tuple[np.ndarray, np.ndarray]:
    """theta -> (R blocks by the truncated series, Q blocks). [CNP], [BD]"""
    Q = skew_from_theta(theta, b, d)
    return cayley_neumann(Q), Q


def materialise(W0: np.ndarray, R: np.ndarray, P: np.ndarray, b_out: int, b_in: int) -> np.ndarray:
    """W = R W0 P with block-diagonal R (on the d_out rows) and P (on the d_in
    columns), computed block by block. This is the weight-centric form that
    the input-centric method avoids on the GPU. [OET], [BD]"""
    W0 = np.asarray(W0, dtype=np.float64)
    m, n = W0.shape
    W = W0.copy()
    for k, (s, r) in enumerate(block_ranges(m, b_out)):
        W[s:s + r, :] = R[k, :r, :r] @ W[s:s + r, :]
    for j, (s, r) in enumerate(block_ranges(n, b_in)):
        W[:, s:s + r] = W[:, s:s + r] @ P[j, :r, :r]
    return W


# ------------------------------------------- block-mixing permutations [PERM]
def permutation_matrix(pi: np.ndarray) -> np.ndarray:
    """The matrix Pi of an index map: (Pi v)_i = v[pi[i]], so row i of Pi is
    the unit row e_pi[i]. [PERM]"""
    pi = np.asarray(pi, dtype=np.int64)
    d = len(pi)
    if sorted(pi.tolist()) != list(range(d)):
        raise ValueError("not a permutation")
    M = np.zeros((d, d))
    M[np.arange(d), pi] = 1.0
    return M


def fold_permutations(W0: np.ndarray, perm_out: np.ndarray, perm_in: np.ndarray) -> np.ndarray:
    """W0' = Pi_out W0 Pi_in^T, i.e. W0'[i][j] = W0[perm_out[i]][perm_in[j]]:
    the two inner permutations of the forward folded into the weight once.
    [PERM] (reduction)"""
    return np.asarray(W0, dtype=np.float64)[np.ix_(np.asarray(perm_out), np.asarray(perm_in))]


def materialise_permuted(W0, R, P, b_out, b_in, perm_out, perm_in):
    """W = Pi_out^T blockdiag(R) Pi_out W0 Pi_in^T blockdiag(P) Pi_in, formed
    as M = blockdiag(R) W0' blockdiag(P) with the folded W0', then
    W[perm_out[i]][perm_in[j]] = M[i][j] (W = Pi_out^T M Pi_in). [PERM], [OET]"""
    M = materialise(fold_permutations(W0, perm_out, perm_in), R, P, b_out, b_in)
    W = np.empty_like(M)
    W[np.ix_(np.asarray(perm_out), np.asarray(perm_in))] = M
    return W


# --------------------------------------------------- INT8 base weight [XQ]
def quantize_rows(W0: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric per-output-row INT8 codes of W0 [d_out, d_in]:
    s_i = amax_i / 127 and q_ij = clamp(rint(w_ij / s_i), -127, 127), every
    operation in float32 (so the codes are decided in the precision the GPU
    uses); a zero row gets s = 0, q = 0. Returns (q int8, s float32). [XQ]"""
    W = np.asarray(W0, dtype=np.float32)
    amax = np.max(np.abs(W), axis=1).astype(np.float32)
    s = (amax / np.float32(127.0)).astype(np.float32)
    q = np.zeros(W.shape, dtype=np.int8)
    for i in range(W.shape[0]):
        if s[i] > 0:
            r = np.rint((W[i] / s[i]).astype(np.float32))
            q[i] = np.clip(r, -127, 127).astype(np.int8)
    return q, s


def dequantize_rows(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W0 = diag(s) q in float64 (exact: an int8 code times a float32). [XQ]"""
    return np.asarray(s, dtype=np.float64)[:, None] * np.asarray(q, dtype=np.float64)


# ------------------------------------------------------- forward / backward
def forward(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """y = W x for every token; token-major Y = X W^T. [OET]"""
    return np.asarray(x, dtype=np.float64) @ W.T


def cayley_vjp(B: np.ndarray, G: np.ndarray) -> np.ndarray:
    """Gradient of the packed generators given G = dL/dR per block.

    R = 2B - I with B = (I - Q)^-1, so dR = 2 B dQ B and
    dL/dQ = 2 B^T G B^T; a packed entry theta_(i,j) enters Q at (i, j) with
    sign + and at (j, i) with sign -, hence
    dL/dtheta_(i,j) = Mx[i, j] - Mx[j, i] with Mx = 2 B^T G B^T.
    (The pages never describe the backward; this is the chain rule.)"""
    b = B.shape[-1]
    iu, ju = packed_upper_index(b)
    out = np.empty((B.shape[0], len(iu)), dtype=np.float64)
    for k in range(B.shape[0]):
        Mx = 2.0 * B[k].T @ G[k] @ B[k].T
        out[k] = Mx[iu, ju] - Mx[ju, iu]
    return out


def _pad_grad_zero(g: np.ndarray, b: int, d: int) -> np.ndarray:
    """Drop (zero) the gradients of padded generator entries."""
    nb = g.shape[0]
    r = d - (nb - 1) * b
    if r < b:
        iu, ju = packed_upper_index(b)
        g = g.copy()
        g[-1, (iu >= r) | (ju >= r)] = 0.0
    return g


def backward(g_y: np.ndarray, x: np.ndarray, W0: np.ndarray,
             R: np.ndarray, B_R: np.ndarray, P: np.ndarray, B_P: np.ndarray,
             b_out: int, b_in: int, vjp=None, perm_out=None,
             perm_in=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Backward of the layer through the materialised weight.

    G_W = g_Y^T X is the gradient of the full weight. With W = R (W0 P):
    dL/dR = G_W (W0 P)^T, of which only the diagonal blocks are parameters;
    with W = (R W0) P: dL/dP = (R W0)^T G_W, again block-diagonal part only.
    Returns (g_x, g_theta_R, g_theta_P). [OET], [BD]; backward derived by the
    chain rule. `vjp(B, G)` maps the block gradients to generator gradients
    (cayley_vjp with B = (I - Q)^-1 by default; cayley_neumann_vjp with
    B = Q for the truncated series).

    With permutations, W = Pi_out^T M Pi_in for M = blockdiag(R) W0'
    blockdiag(P): the gradient of M is G_M = Pi_out G_W Pi_in^T
    (G_M[i][j] = G_W[perm_out[i]][perm_in[j]]) and the blocks see W0' in
    place of W0. [PERM]"""
    vjp = cayley_vjp if vjp is None else vjp
    g_y = np.asarray(g_y, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    W0 = np.asarray(W0, dtype=np.float64)
    m, n = W0.shape
    permuted = perm_out is not None
    if permuted:
        W = materialise_permuted(W0, R, P, b_out, b_in, perm_out, perm_in)
    else:
        W = materialise(W0, R, P, b_out, b_in)
    g_x = g_y @ W
    G_W = g_y.T @ x
    if permuted:
        G_W = G_W[np.ix_(np.asarray(perm_out), np.asarray(perm_in))]
        W0 = fold_permutations(W0, perm_out, perm_in)
    ident_R = np.broadcast_to(np.eye(b_out), R.shape)
    ident_P = np.broadcast_to(np.eye(b_in), P.shape)
    W0P = materialise(W0, ident_R, P, b_out, b_in)
    RW0 = materialise(W0, R, ident_P, b_out, b_in)
    G_R = np.zeros_like(R)
    for k, (s, r) in enumerate(block_ranges(m, b_out)):
        G_R[k, :r, :r] = G_W[s:s + r, :] @ W0P[s:s + r, :].T
    G_P = np.zeros_like(P)
    for j, (s, r) in enumerate(block_ranges(n, b_in)):
        G_P[j, :r, :r] = RW0[:, s:s + r].T @ G_W[:, s:s + r]
    g_tR = _pad_grad_zero(vjp(B_R, G_R), b_out, m)
    g_tP = _pad_grad_zero(vjp(B_P, G_P), b_in, n)
    return g_x, g_tR, g_tP


# ----------------------------------------- second route: input-centric [IC]
def _apply_blocks(a: np.ndarray, blocks: np.ndarray, b: int, transpose: bool) -> np.ndarray:
    """Token-major block-diagonal product: out[:, blk] = a[:, blk] M^T for
    M = blocks[k] (transpose=True) or a[:, blk] M (transpose=False)."""
    out = np.empty_like(a)
    for k, (s, r) in enumerate(block_ranges(a.shape[1], b)):
        M = blocks[k, :r, :r]
        out[:, s:s + r] = a[:, s:s + r] @ (M.T if transpose else M)
    return out


def forward_input_centric(x, W0, R, P, b_out, b_in, perm_out=None, perm_in=None):
    """U = X P^T, Z = U W0^T, Y = Z R^T (token-major). Returns (Y, Z, U). [IC]
    With permutations (W0 is then the folded W0'): X_p = X[:, perm_in]
    (gather), U = X_p blockdiag(P)^T, Z = U W0'^T, Y_p = Z blockdiag(R)^T and
    Y[:, perm_out] = Y_p (scatter). [PERM]"""
    x = np.asarray(x, dtype=np.float64)
    if perm_in is not None:
        x = x[:, np.asarray(perm_in)]
    U = _apply_blocks(x, P, b_in, transpose=True)
    Z = U @ np.asarray(W0, dtype=np.float64).T
    Y = _apply_blocks(Z, R, b_out, transpose=True)
    if perm_out is not None:
        Yp = Y
        Y = np.empty_like(Yp)
        Y[:, np.asarray(perm_out)] = Yp
    return Y, Z, U


def backward_input_centric(g_y, x, W0, R, B_R, P, B_P, b_out, b_in, vjp=None,
                           perm_out=None, perm_in=None):
    """Backward along the input-centric dataflow:
    g_Z = g_Y R, G_R[k] = g_Y[:, k]^T Z[:, k], g_U = g_Z W0,
    G_P[j] = g_U[:, j]^T X[:, j], g_X = g_U P. [IC], chain rule.
    With permutations (W0 folded): g_Y and X are gathered by perm_out and
    perm_in first and g_X is scattered by perm_in at the end. [PERM]"""
    vjp = cayley_vjp if vjp is None else vjp
    g_y = np.asarray(g_y, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    W0 = np.asarray(W0, dtype=np.float64)
    m, n = W0.shape
    if perm_out is not None:
        g_y = g_y[:, np.asarray(perm_out)]
    if perm_in is not None:
        x = x[:, np.asarray(perm_in)]
    _, Z, _ = forward_input_centric(x, W0, R, P, b_out, b_in)
    g_Z = _apply_blocks(g_y, R, b_out, transpose=False)
    G_R = np.zeros_like(R)
    for k, (s, r) in enumerate(block_ranges(m, b_out)):
        G_R[k, :r, :r] = g_y[:, s:s + r].T @ Z[:, s:s + r]
    g_U = g_Z @ W0
    G_P = np.zeros_like(P)
    for j, (s, r) in enumerate(block_ranges(n, b_in)):
        G_P[j, :r, :r] = g_U[:, s:s + r].T @ x[:, s:s + r]
    g_x = _apply_blocks(g_U, P, b_in, transpose=False)
    if perm_in is not None:
        g_xp = g_x
        g_x = np.empty_like(g_xp)
        g_x[:, np.asarray(perm_in)] = g_xp
    g_tR = _pad_grad_zero(vjp(B_R, G_R), b_out, m)
    g_tP = _pad_grad_zero(vjp(B_P, G_P), b_in, n)
    return g_x, g_tR, g_tP


class LayerOracle:
    """One layer's full oracle result (orthogonal build, forward, backward),
    computed through the materialised weight. map: "cayley" (exact) or "cnp"
    (truncated Cayley-Neumann series); B_R / B_P hold what that map's VJP
    needs ((I - Q)^-1 or Q). perm_out / perm_in: optional block-mixing index
    maps of R and P (both or neither); W0 is the unfolded weight."""

    def __init__(self, W0, theta_R, theta_P, b_out, b_in, map="cayley", perm_out=None,
                 perm_in=None):
        self.W0 = np.asarray(W0, dtype=np.float64)
        m, n = self.W0.shape
        self.b_out, self.b_in = b_out, b_in
        if map not in ("cayley", "cnp"):
            raise ValueError(f"unknown orthogonal map {map!r}")
        build = orthogonal_blocks if map == "cayley" else orthogonal_blocks_cnp
        self.vjp = cayley_vjp if map == "cayley" else cayley_neumann_vjp
        self.R, self.B_R = build(theta_R, b_out, m)
        self.P, self.B_P = build(theta_P, b_in, n)
        if (perm_out is None) != (perm_in is None):
            raise ValueError("give both permutations or neither")
        self.perm_out, self.perm_in = perm_out, perm_in
        if perm_out is None:
            self.W = materialise(self.W0, self.R, self.P, b_out, b_in)
        else:
            self.W = materialise_permuted(self.W0, self.R, self.P, b_out, b_in, perm_out, perm_in)

    def forward(self, x):
        return forward(x, self.W)

    def backward(self, g_y, x):
        return backward(g_y, x, self.W0, self.R, self.B_R, self.P, self.B_P,
                        self.b_out, self.b_in, self.vjp, self.perm_out, self.perm_in)
