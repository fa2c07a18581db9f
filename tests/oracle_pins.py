"""Pins of the float64 oracle against facts fixed outside it.

Each pin_* function raises AssertionError when the oracle disagrees with a
closed form, an invariant, a textbook routine or finite differences. The pins
are collected by tests/test_oracle.py and re-run there against planted
mistakes (tests/test_oracle_mutations.py) to show each mistake is caught.
"""
from __future__ import annotations

import math
import os

import numpy as np
import scipy.linalg

import oracle.poetx_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_closed_forms():
    cases = []
    with open(os.path.join(GOLDEN, "cayley_closed_forms.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, b, th, R = [c.strip() for c in line.split("|")]
            b = int(b)
            theta = np.array([float(v) for v in th.split(",")])
            Rm = np.array([float(v) for v in R.split(",")]).reshape(b, b)
            cases.append((name, b, theta, Rm))
    return cases


# ----------------------------------------------------------------- packing
def pin_packing_order():
    """Packed position p of (i, j) is i(2b - i - 1)/2 + (j - i - 1)."""
    for b in (2, 3, 5, 8):
        iu, ju = O.packed_upper_index(b)
        assert len(iu) == b * (b - 1) // 2
        for p, (i, j) in enumerate(zip(iu, ju)):
            assert i < j
            assert p == i * (2 * b - i - 1) // 2 + (j - i - 1)
    rng = np.random.default_rng(1)
    th = rng.standard_normal((3, 10))
    Q = O.skew_from_theta(th, 5)
    assert np.array_equal(Q, -np.transpose(Q, (0, 2, 1)))
    assert np.all(np.diagonal(Q, axis1=1, axis2=2) == 0)
    assert np.array_equal(O.theta_from_skew(Q), th)
    # an entry lands where the formula says: theta position 5 of b=4 is (2, 3)
    th4 = np.zeros((1, 6)); th4[0, 5] = 7.0
    Q4 = O.skew_from_theta(th4, 4)
    assert Q4[0, 2, 3] == 7.0 and Q4[0, 3, 2] == -7.0 and np.count_nonzero(Q4) == 2


# ----------------------------------------------------------- closed forms
def pin_golden_closed_forms(tol=1e-15):
    for name, b, theta, Rref in load_closed_forms():
        R, _ = O.orthogonal_blocks(theta[None, :], b, b)
        err = np.max(np.abs(R[0] - Rref))
        assert err <= tol * 4, (name, err)


def pin_b2_rotation():
    """b = 2, theta = t: rotation by phi = 2 atan t, R = [[c, s], [-s, c]]."""
    for t in np.linspace(-5, 5, 41):
        R, _ = O.orthogonal_blocks(np.array([[t]]), 2, 2)
        phi = 2.0 * math.atan(t)
        ref = np.array([[math.cos(phi), math.sin(phi)], [-math.sin(phi), math.cos(phi)]])
        assert np.max(np.abs(R[0] - ref)) < 1e-14, t


def _cross(w):
    return np.array([[0, -w[2], w[1]], [w[2], 0, -w[0]], [-w[1], w[0], 0]], dtype=np.float64)


def pin_b3_rodrigues():
    """b = 3: Q = [w]_x maps to the rotation about w by 2 atan|w| (Rodrigues'
    formula R = I + sin(phi) K + (1 - cos(phi)) K^2, K = [w/|w|]_x)."""
    rng = np.random.default_rng(3)
    for _ in range(20):
        w = rng.standard_normal(3) * rng.uniform(0.05, 3.0)
        theta = np.array([[-w[2], w[1], -w[0]]])  # Q01 = -w3, Q02 = w2, Q12 = -w1
        Q = O.skew_from_theta(theta, 3)[0]
        assert np.allclose(Q, _cross(w), atol=0, rtol=0)
        R, _ = O.orthogonal_blocks(theta, 3, 3)
        nw = np.linalg.norm(w)
        K = _cross(w / nw)
        phi = 2.0 * math.atan(nw)
        ref = np.eye(3) + math.sin(phi) * K + (1 - math.cos(phi)) * (K @ K)
        assert np.max(np.abs(R[0] - ref)) < 1e-13


def pin_eigenvalue_map():
    """Q with eigenvalues +-i lambda_k maps to R with eigenvalues
    exp(+-2i atan lambda_k): build Q = V diag(2x2 generators) V^T."""
    rng = np.random.default_rng(5)
    b = 8
    lam = np.array([0.1, 0.7, 1.5, 4.0])
    D = np.zeros((b, b))
    for k, l in enumerate(lam):
        D[2 * k, 2 * k + 1] = l
        D[2 * k + 1, 2 * k] = -l
    V, _ = np.linalg.qr(rng.standard_normal((b, b)))
    Q = V @ D @ V.T
    R, _ = O.cayley(Q[None])
    ev = np.linalg.eigvals(R[0])
    ang = np.sort(np.abs(np.angle(ev)))
    ref = np.sort(np.concatenate([2 * np.arctan(lam)] * 2))
    assert np.max(np.abs(ang - ref)) < 1e-12
    assert np.max(np.abs(np.abs(ev) - 1)) < 1e-12


# ------------------------------------------------------------- invariants
def pin_orthogonality_det_transpose():
    rng = np.random.default_rng(7)
    for b, sigma in ((4, 0.3), (32, 0.02), (64, 0.5), (256, 0.01)):
        th = rng.standard_normal((3, b * (b - 1) // 2)) * sigma
        R, _ = O.orthogonal_blocks(th, b, 3 * b)
        I = np.eye(b)
        for k in range(3):
            assert np.linalg.norm(R[k].T @ R[k] - I) <= 1e-10
            assert abs(np.linalg.det(R[k]) - 1.0) <= 1e-10
        Rm, _ = O.orthogonal_blocks(-th, b, 3 * b)
        assert np.max(np.abs(Rm - np.transpose(R, (0, 2, 1)))) <= 1e-12
        R0, _ = O.orthogonal_blocks(np.zeros_like(th), b, 3 * b)
        assert np.array_equal(R0, np.broadcast_to(I, R0.shape))
        # inverse Cayley (R - I)(R + I)^-1 gives back Q
        Q = O.skew_from_theta(th, b)
        for k in range(3):
            Qb = (R[k] - I) @ np.linalg.inv(R[k] + I)
            assert np.max(np.abs(Qb - Q[k])) <= 1e-10 * max(1.0, np.abs(Q[k]).max())


def pin_spectrum(m=384, n=256, b=64, sigma=0.05, seed=11):
    """Singular values of R W0 P equal those of W0 (orthogonal equivalence)."""
    rng = np.random.default_rng(seed)
    W0 = rng.standard_normal((m, n)) / math.sqrt(n)
    thR = rng.standard_normal((-(-m // b), b * (b - 1) // 2)) * sigma
    thP = rng.standard_normal((-(-n // b), b * (b - 1) // 2)) * sigma
    ora = O.LayerOracle(W0, thR, thP, b, b)
    s = np.linalg.svd(ora.W, compute_uv=False)
    s0 = np.linalg.svd(W0, compute_uv=False)
    assert np.max(np.abs(s - s0)) / s0[0] <= 1e-9
    assert np.max(np.abs(ora.W - W0)) > 1e-3  # the transform is not trivial


def pin_dense_block_diag(m=20, n=12, b_out=8, b_in=8, seed=13):
    """W equals the dense product R_dense W0 P_dense, with the dense matrices
    assembled by scipy.linalg.block_diag from independently computed blocks
    R_k = (I - Q_k)^-1 (I + Q_k) (the commuted form). Sizes include ragged
    last blocks (20 = 8 + 8 + 4, 12 = 8 + 4)."""
    rng = np.random.default_rng(seed)
    W0 = rng.standard_normal((m, n))
    thR = rng.standard_normal((-(-m // b_out), b_out * (b_out - 1) // 2)) * 0.3
    thP = rng.standard_normal((-(-n // b_in), b_in * (b_in - 1) // 2)) * 0.3

    def dense(theta, b, d):
        iu, ju = np.triu_indices(b, k=1)
        blocks = []
        for k, s in enumerate(range(0, d, b)):
            r = min(b, d - s)
            Q = np.zeros((b, b))
            Q[iu, ju] = theta[k]
            Q = Q - Q.T
            Qr = Q[:r, :r]
            I = np.eye(r)
            blocks.append(scipy.linalg.solve(I - Qr, I + Qr))
        return scipy.linalg.block_diag(*blocks)

    Rd, Pd = dense(thR, b_out, m), dense(thP, b_in, n)
    ora = O.LayerOracle(W0, thR, thP, b_out, b_in)
    assert np.max(np.abs(ora.W - Rd @ W0 @ Pd)) <= 1e-12


def _layer(m, n, b_out, b_in, N, sigma, seed):
    rng = np.random.default_rng(seed)
    W0 = rng.standard_normal((m, n)) / math.sqrt(n)
    thR = rng.standard_normal((-(-m // b_out), b_out * (b_out - 1) // 2)) * sigma
    thP = rng.standard_normal((-(-n // b_in), b_in * (b_in - 1) // 2)) * sigma
    x = rng.standard_normal((N, n))
    g_y = rng.standard_normal((N, m))
    return W0, thR, thP, x, g_y


def pin_input_centric_equals_materialised():
    for (m, n, b_out, b_in, N) in ((96, 64, 32, 16, 7), (100, 72, 32, 32, 9)):
        W0, thR, thP, x, g_y = _layer(m, n, b_out, b_in, N, 0.2, 17)
        ora = O.LayerOracle(W0, thR, thP, b_out, b_in)
        y = ora.forward(x)
        y2, _, _ = O.forward_input_centric(x, W0, ora.R, ora.P, b_out, b_in)
        assert np.max(np.abs(y - y2)) <= 1e-12 * np.abs(y).max()
        g1 = ora.backward(g_y, x)
        g2 = O.backward_input_centric(g_y, x, W0, ora.R, ora.B_R, ora.P, ora.B_P, b_out, b_in)
        for a, c in zip(g1, g2):
            assert np.max(np.abs(a - c)) <= 1e-12 * max(np.abs(a).max(), 1e-300)


def pin_theta_zero():
    """theta = 0: y = x W0^T (plain numpy GEMM) and g_theta = 2 (G - G^T)
    packed, with G the block of g_y^T (x W0^T) (R) or (g_y W0)^T x (P)."""
    m, n, b, N = 48, 32, 16, 6
    W0, thR, thP, x, g_y = _layer(m, n, b, b, N, 0.0, 19)
    ora = O.LayerOracle(W0, thR, thP, b, b)
    assert np.max(np.abs(ora.forward(x) - x @ W0.T)) <= 1e-13
    g_x, gR, gP = ora.backward(g_y, x)
    assert np.max(np.abs(g_x - g_y @ W0)) <= 1e-13
    iu, ju = np.triu_indices(b, k=1)
    Zf = x @ W0.T
    gU = g_y @ W0
    for k in range(m // b):
        G = g_y[:, k * b:(k + 1) * b].T @ Zf[:, k * b:(k + 1) * b]
        assert np.max(np.abs(gR[k] - 2 * (G[iu, ju] - G[ju, iu]))) <= 1e-12
    for j in range(n // b):
        G = gU[:, j * b:(j + 1) * b].T @ x[:, j * b:(j + 1) * b]
        assert np.max(np.abs(gP[j] - 2 * (G[iu, ju] - G[ju, iu]))) <= 1e-12


def pin_vjp_forms():
    """2 B^T G B^T equals 1/2 (R^T + I) G (R^T + I) (R = 2B - I)."""
    rng = np.random.default_rng(23)
    b = 16
    th = rng.standard_normal((2, b * (b - 1) // 2)) * 0.4
    R, B = O.orthogonal_blocks(th, b, 2 * b)
    G = rng.standard_normal((2, b, b))
    I = np.eye(b)
    for k in range(2):
        a = 2 * B[k].T @ G[k] @ B[k].T
        c = 0.5 * (R[k].T + I) @ G[k] @ (R[k].T + I)
        assert np.max(np.abs(a - c)) <= 1e-13 * np.abs(a).max()


def pin_adjoint():
    """<g_y, x W^T> = <g_y W, x>: g_x is the adjoint of the forward map."""
    W0, thR, thP, x, g_y = _layer(40, 24, 8, 8, 5, 0.3, 29)
    ora = O.LayerOracle(W0, thR, thP, 8, 8)
    g_x, _, _ = ora.backward(g_y, x)
    lhs = np.sum(g_y * ora.forward(x))
    rhs = np.sum(g_x * x)
    assert abs(lhs - rhs) <= 1e-12 * abs(lhs)


def pin_finite_differences(m=8, n=8, b=4, N=5, seed=31, h=1e-6, rtol=1e-6):
    """Central differences of L = <g_y, y(x, theta_R, theta_P)> in float64
    against the oracle's backward, for every theta and x entry."""
    W0, thR, thP, x, g_y = _layer(m, n, b, b, N, 0.3, seed)

    def loss(thR_, thP_, x_):
        return float(np.sum(g_y * O.LayerOracle(W0, thR_, thP_, b, b).forward(x_)))

    g_x, gR, gP = O.LayerOracle(W0, thR, thP, b, b).backward(g_y, x)

    def fd(arr, fn):
        out = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a1 = arr.copy(); a1[idx] += h
            a2 = arr.copy(); a2[idx] -= h
            out[idx] = (fn(a1) - fn(a2)) / (2 * h)
        return out

    fR = fd(thR, lambda a: loss(a, thP, x))
    fP = fd(thP, lambda a: loss(thR, a, x))
    fx = fd(x, lambda a: loss(thR, thP, a))
    for got, ref in ((gR, fR), (gP, fP), (g_x, fx)):
        scale = np.abs(ref).max()
        assert np.max(np.abs(got - ref)) <= rtol * scale, (np.max(np.abs(got - ref)), scale)


def pin_padding_gradients():
    """With b not dividing d, the padded generator entries do not change the
    output: their FD gradient is 0 and the oracle reports 0 for them; the
    other entries still match FD."""
    m, n, b, N = 10, 6, 4, 3
    W0, thR, thP, x, g_y = _layer(m, n, b, b, N, 0.3, 37)

    def loss(thR_, thP_):
        return float(np.sum(g_y * O.LayerOracle(W0, thR_, thP_, b, b).forward(x)))

    _, gR, gP = O.LayerOracle(W0, thR, thP, b, b).backward(g_y, x)
    h = 1e-6
    for th, g, which in ((thR, gR, 0), (thP, gP, 1)):
        for idx in np.ndindex(th.shape):
            a1 = th.copy(); a1[idx] += h
            a2 = th.copy(); a2[idx] -= h
            if which == 0:
                f = (loss(a1, thP) - loss(a2, thP)) / (2 * h)
            else:
                f = (loss(thR, a1) - loss(thR, a2)) / (2 * h)
            assert abs(g[idx] - f) <= 1e-6 * max(1.0, abs(f)), (which, idx, g[idx], f)
    iu, ju = O.packed_upper_index(b)
    pad_R = (iu >= m - 2 * b) | (ju >= m - 2 * b)
    assert np.all(gR[-1, pad_R] == 0.0) and np.any(pad_R)


# ------------------------------------------ Cayley-Neumann series (CNP)
def load_cnp_closed_forms():
    """(kind, name, b, theta, values, grad) rows of the hand-derived CNP file."""
    rows = []
    with open(os.path.join(GOLDEN, "cnp_closed_forms.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = [c.strip() for c in line.split("|")]
            kind, name, b, th = parts[0], parts[1], int(parts[2]), parts[3]
            theta = np.array([float(v) for v in th.split(",")])
            vals = np.array([float(v) for v in parts[4].split(",")]).reshape(b, b)
            grad = float(parts[5]) if kind == "G" else None
            rows.append((kind, name, b, theta, vals, grad))
    return rows


def pin_cnp_golden(tol=1e-15):
    """The truncated series and its derivative on the hand-derived b = 2 and
    b = 4 cases (values exact in binary or within a few ulps)."""
    rows = load_cnp_closed_forms()
    assert sum(r[0] == "R" for r in rows) >= 6 and sum(r[0] == "G" for r in rows) >= 4
    for kind, name, b, theta, vals, grad in rows:
        Q = O.skew_from_theta(theta[None, :], b)
        if kind == "R":
            R = O.cayley_neumann(Q)[0]
            scale = max(1.0, np.abs(vals).max())
            assert np.max(np.abs(R - vals)) <= 8 * tol * scale, (name, R, vals)
        else:
            g = O.cayley_neumann_vjp(Q, vals[None])[0]
            assert g.shape == (1,) and abs(g[0] - grad) <= 1e-14, (name, g, grad)


def pin_cnp_b3_closed_form():
    """b = 3: Q = [w]_x has Q^3 = -|w|^2 Q and Q^4 = -|w|^2 Q^2, so the series
    is R = I + 2 (1 - |w|^2)(Q + Q^2), with Q^2 = w w^T - |w|^2 I."""
    rng = np.random.default_rng(41)
    for _ in range(20):
        w = rng.standard_normal(3) * rng.uniform(0.05, 1.5)
        # theta order (0,1), (0,2), (1,2) holds Q entries -w2, w1, -w0
        theta = np.array([[-w[2], w[1], -w[0]]])
        K = _cross(w)
        n2 = float(w @ w)
        K2 = np.outer(w, w) - n2 * np.eye(3)
        ref = np.eye(3) + 2.0 * (1.0 - n2) * (K + K2)
        R = O.cayley_neumann(O.skew_from_theta(theta, 3))[0]
        assert np.max(np.abs(R - ref)) <= 1e-13 * max(1.0, np.abs(ref).max()), (w, R, ref)


def pin_cnp_series_tail():
    """Exact map minus truncated series is the tail 2 sum_{k>=5} Q^k =
    2 Q^5 (I - Q)^-1, computed from the (separately pinned) exact map and an
    independent solve; at small |Q| the two maps agree to O(|Q|^5)."""
    rng = np.random.default_rng(43)
    for b, sigma in ((5, 0.3), (16, 0.05), (32, 0.02), (7, 0.6)):
        th = rng.standard_normal((3, b * (b - 1) // 2)) * sigma
        Q = O.skew_from_theta(th, b)
        R_exact, _ = O.cayley(Q)
        R_cnp = O.cayley_neumann(Q)
        for k in range(3):
            tail = 2.0 * np.linalg.matrix_power(Q[k], 5) @ np.linalg.solve(np.eye(b) - Q[k], np.eye(b))
            diff = R_exact[k] - R_cnp[k]
            assert np.max(np.abs(diff - tail)) <= 1e-13 * max(1.0, np.abs(tail).max()), (b, sigma)
            assert np.abs(tail).max() > 0.0


def pin_cnp_vjp_frechet():
    """The VJP of a real matrix polynomial p at Q is the Frechet derivative of
    p at Q^T in the direction G: the upper-right block of p applied to the
    block-triangular [[Q^T, G], [0, Q^T]]. Evaluated with the series itself
    (independently of the VJP's double sum), then packed."""
    rng = np.random.default_rng(47)
    for b, sigma in ((4, 0.5), (9, 0.2), (16, 0.1)):
        th = rng.standard_normal((2, b * (b - 1) // 2)) * sigma
        Q = O.skew_from_theta(th, b)
        G = rng.standard_normal((2, b, b))
        got = O.cayley_neumann_vjp(Q, G)
        iu, ju = O.packed_upper_index(b)
        for k in range(2):
            M = np.zeros((2 * b, 2 * b))
            M[:b, :b] = Q[k].T
            M[b:, b:] = Q[k].T
            M[:b, b:] = G[k]
            D = O.cayley_neumann(M[None])[0][:b, b:]
            ref = D[iu, ju] - D[ju, iu]
            assert np.max(np.abs(got[k] - ref)) <= 1e-13 * np.abs(ref).max(), (b, k)


def pin_cnp_theta_zero():
    """theta = 0: the series gives R = I and the same generator gradient as
    the exact map, 2 (G - G^T) packed."""
    rng = np.random.default_rng(53)
    b = 8
    Q = np.zeros((3, b, b))
    G = rng.standard_normal((3, b, b))
    assert np.array_equal(O.cayley_neumann(Q), np.broadcast_to(np.eye(b), Q.shape))
    iu, ju = O.packed_upper_index(b)
    ref = 2.0 * (G[:, iu, ju] - G[:, ju, iu])
    assert np.max(np.abs(O.cayley_neumann_vjp(Q, G) - ref)) <= 1e-14


def pin_cnp_finite_differences(h=1e-6, rtol=1e-6):
    """Central differences of L = <g_y, y> for the layer built with the
    series, against the oracle's backward, for every generator and x entry;
    with b dividing d and (second case) with a padded last block, whose
    padded entries must have zero gradient."""
    for (m, n, b, N, seed) in ((8, 8, 4, 5, 59), (10, 6, 4, 3, 61)):
        W0, thR, thP, x, g_y = _layer(m, n, b, b, N, 0.3, seed)

        def loss(thR_, thP_, x_):
            return float(np.sum(g_y * O.LayerOracle(W0, thR_, thP_, b, b, map="cnp").forward(x_)))

        g_x, gR, gP = O.LayerOracle(W0, thR, thP, b, b, map="cnp").backward(g_y, x)

        def fd(arr, fn):
            out = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                a1 = arr.copy(); a1[idx] += h
                a2 = arr.copy(); a2[idx] -= h
                out[idx] = (fn(a1) - fn(a2)) / (2 * h)
            return out

        fR = fd(thR, lambda a: loss(a, thP, x))
        fP = fd(thP, lambda a: loss(thR, a, x))
        fx = fd(x, lambda a: loss(thR, thP, a))
        for got, ref in ((gR, fR), (gP, fP), (g_x, fx)):
            scale = np.abs(ref).max()
            assert np.max(np.abs(got - ref)) <= rtol * scale, (np.max(np.abs(got - ref)), scale)
        if m % b:
            iu, ju = O.packed_upper_index(b)
            r = m - (gR.shape[0] - 1) * b
            pad = (iu >= r) | (ju >= r)
            assert np.all(gR[-1, pad] == 0.0) and np.any(pad)
            R = O.LayerOracle(W0, thR, thP, b, b, map="cnp").R
            assert np.array_equal(R[-1, r:, r:], np.eye(b - r))


# ------------------------------------------- block-mixing permutations
def _perm_layer(m, n, b, N, sigma, seed):
    W0, thR, thP, x, g_y = _layer(m, n, b, b, N, sigma, seed)
    rng = np.random.default_rng(seed + 1000)
    return W0, thR, thP, x, g_y, rng.permutation(m), rng.permutation(n)


def pin_permutation_convention():
    """(Pi v)_i = v[pi(i)] on a hand example, and non-permutations refused."""
    Pi = O.permutation_matrix(np.array([2, 0, 1]))
    assert np.array_equal(Pi @ np.array([10.0, 20.0, 30.0]), np.array([30.0, 10.0, 20.0]))
    assert np.array_equal(Pi @ Pi.T, np.eye(3))
    for bad in ([0, 0, 1], [0, 1, 3]):
        try:
            O.permutation_matrix(np.array(bad))
        except ValueError:
            continue
        raise AssertionError(f"accepted {bad}")


def pin_perm_explicit_matrices():
    """The permuted layer equals the explicit product with permutation and
    block-diagonal matrices (scipy block_diag), and the fold equals
    Pi_R W0 Pi_P^T as a matrix product."""
    for (m, n, b, seed) in ((24, 16, 8, 71), (20, 12, 8, 73)):   # second: padded blocks
        W0, thR, thP, x, _, po, pi = _perm_layer(m, n, b, 4, 0.3, seed)
        ora = O.LayerOracle(W0, thR, thP, b, b, perm_out=po, perm_in=pi)
        PiR, PiP = O.permutation_matrix(po), O.permutation_matrix(pi)
        DR = scipy.linalg.block_diag(*[ora.R[k, :r, :r] for k, (_, r) in enumerate(O.block_ranges(m, b))])
        DP = scipy.linalg.block_diag(*[ora.P[j, :r, :r] for j, (_, r) in enumerate(O.block_ranges(n, b))])
        W = PiR.T @ DR @ PiR @ W0 @ PiP.T @ DP @ PiP
        assert np.max(np.abs(ora.W - W)) <= 1e-13
        assert np.max(np.abs(ora.forward(x) - x @ W.T)) <= 1e-12
        assert np.max(np.abs(O.fold_permutations(W0, po, pi) - PiR @ W0 @ PiP.T)) == 0.0


def pin_perm_identity_reduces():
    """Identity index maps give exactly the unpermuted layer."""
    m, n, b = 32, 24, 8
    W0, thR, thP, x, g_y = _layer(m, n, b, b, 5, 0.3, 79)
    a = O.LayerOracle(W0, thR, thP, b, b)
    c = O.LayerOracle(W0, thR, thP, b, b, perm_out=np.arange(m), perm_in=np.arange(n))
    assert np.array_equal(a.W, c.W)
    for u, v in zip(a.backward(g_y, x), c.backward(g_y, x)):
        assert np.array_equal(u, v)


def pin_perm_spectrum_and_routes():
    """With permutations R and P stay orthogonal, so W keeps W0's singular
    values; the input-centric route (gather, blocks, folded W0, blocks,
    scatter) equals the materialised one, forward and backward."""
    m, n, b, N = 48, 40, 8, 7
    W0, thR, thP, x, g_y, po, pi = _perm_layer(m, n, b, N, 0.4, 83)
    ora = O.LayerOracle(W0, thR, thP, b, b, perm_out=po, perm_in=pi)
    s0 = np.linalg.svd(W0, compute_uv=False)
    s1 = np.linalg.svd(ora.W, compute_uv=False)
    assert np.max(np.abs(s0 - s1)) <= 1e-12 * s0.max()
    W0f = O.fold_permutations(W0, po, pi)
    y2, _, _ = O.forward_input_centric(x, W0f, ora.R, ora.P, b, b, po, pi)
    assert np.max(np.abs(ora.forward(x) - y2)) <= 1e-12
    g1 = ora.backward(g_y, x)
    g2 = O.backward_input_centric(g_y, x, W0f, ora.R, ora.B_R, ora.P, ora.B_P, b, b, None, po, pi)
    for u, v in zip(g1, g2):
        assert np.max(np.abs(u - v)) <= 1e-12 * max(np.abs(u).max(), 1e-300)


def pin_perm_finite_differences(h=1e-6, rtol=1e-6):
    """Central differences of L = <g_y, y> for the permuted layer (exact map
    and series) against the oracle's backward, every generator and x entry."""
    for map_ in ("cayley", "cnp"):
        m, n, b, N = 8, 12, 4, 4
        W0, thR, thP, x, g_y, po, pi = _perm_layer(m, n, b, N, 0.3, 89)

        def loss(thR_, thP_, x_):
            o = O.LayerOracle(W0, thR_, thP_, b, b, map=map_, perm_out=po, perm_in=pi)
            return float(np.sum(g_y * o.forward(x_)))

        g_x, gR, gP = O.LayerOracle(W0, thR, thP, b, b, map=map_, perm_out=po,
                                    perm_in=pi).backward(g_y, x)

        def fd(arr, fn):
            out = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                a1 = arr.copy(); a1[idx] += h
                a2 = arr.copy(); a2[idx] -= h
                out[idx] = (fn(a1) - fn(a2)) / (2 * h)
            return out

        for got, ref in ((gR, fd(thR, lambda a: loss(a, thP, x))),
                         (gP, fd(thP, lambda a: loss(thR, a, x))),
                         (g_x, fd(x, lambda a: loss(thR, thP, a)))):
            assert np.max(np.abs(got - ref)) <= rtol * np.abs(ref).max(), map_


# ------------------------------------------------------------ INT8 weights
def pin_quantize_closed_forms():
    """Rows built as 2^-7 times integers with amax 127 * 2^-7 quantise to
    exactly those integers with s = 2^-7; ties w / s = k + 1/2 round to even;
    a zero row gives s = 0, q = 0; rows are scaled independently."""
    u = 2.0 ** -7
    W = np.zeros((4, 8))
    W[0] = u * np.array([127, -3, 64, 0, 1, -127, 5, 100])
    W[1] = u * np.array([2.5, 3.5, -2.5, -3.5, 0.5, 1.5, 127, 0])   # ties
    W[3] = 0.5 * u * np.array([127, 1, 2, 3, -4, 5, 6, 7])          # s = 2^-8
    q, s = O.quantize_rows(W)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert s[0] == u and s[1] == u and s[2] == 0.0 and s[3] == u / 2
    assert np.array_equal(q[0], [127, -3, 64, 0, 1, -127, 5, 100])
    assert np.array_equal(q[1], [2, 4, -2, -4, 0, 2, 127, 0])
    assert np.array_equal(q[2], np.zeros(8))
    assert np.array_equal(q[3], [127, 1, 2, 3, -4, 5, 6, 7])
    D = O.dequantize_rows(q, s)
    assert np.array_equal(D[0], W[0]) and np.array_equal(D[3], W[3])
    assert np.array_equal(D[1], u * np.array([2, 4, -2, -4, 0, 2, 127, 0]))
    assert np.array_equal(D[2], np.zeros(8))


def pin_quantize_error_bound():
    """Random rows: |q| <= 127 with 127 reached in every nonzero row, and
    |w - s q| <= s / 2 up to float32 rounding of w / s."""
    rng = np.random.default_rng(97)
    W = (rng.standard_normal((64, 300)) * rng.uniform(0.01, 3.0, (64, 1))).astype(np.float32)
    q, s = O.quantize_rows(W)
    assert np.all(np.abs(q.astype(int)) <= 127)
    assert np.all(np.max(np.abs(q.astype(int)), axis=1) == 127)
    err = np.abs(W.astype(np.float64) - O.dequantize_rows(q, s))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-5)), err.max()


ALL_PINS = [
    pin_packing_order, pin_golden_closed_forms, pin_b2_rotation, pin_b3_rodrigues,
    pin_eigenvalue_map, pin_orthogonality_det_transpose, pin_spectrum,
    pin_dense_block_diag, pin_input_centric_equals_materialised, pin_theta_zero,
    pin_vjp_forms, pin_adjoint, pin_finite_differences, pin_padding_gradients,
    pin_cnp_golden, pin_cnp_b3_closed_form, pin_cnp_series_tail, pin_cnp_vjp_frechet,
    pin_cnp_theta_zero, pin_cnp_finite_differences, pin_permutation_convention,
    pin_perm_explicit_matrices, pin_perm_identity_reduces, pin_perm_spectrum_and_routes,
    pin_perm_finite_differences, pin_quantize_closed_forms, pin_quantize_error_bound,
]
