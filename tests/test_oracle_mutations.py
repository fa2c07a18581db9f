"""Planted mistakes in the oracle (on the CPU) must each fail a pin.

Each case rewrites one line of an oracle function (a dropped term, a wrong
sign or index, a transposed operand), installs the rewritten function in the
oracle module for the duration of the test, and checks that the named pins
no longer all pass. This shows the pins constrain every part of the oracle.
"""
import inspect
import textwrap

import pytest

import oracle.poetx_oracle as O
from tests import oracle_pins as pins

MUTATIONS = [
    # (function, original text, planted text, pins expected to catch it)
    ("cayley", "(I + q) @ bk", "(I - q) @ np.linalg.inv(I + q)",
     [pins.pin_b3_rodrigues, pins.pin_golden_closed_forms]),
    ("cayley", "(I + q) @ bk", "q @ bk", [pins.pin_b2_rotation]),
    ("packed_upper_index", "for i in range(b):\n        for j in range(i + 1, b):",
     "for j in range(b):\n        for i in range(j):", [pins.pin_packing_order, pins.pin_golden_closed_forms]),
    ("skew_from_theta", "Q[:, ju, iu] = -theta", "Q[:, ju, iu] = theta",
     [pins.pin_packing_order, pins.pin_orthogonality_det_transpose]),
    ("cayley_vjp", "Mx = 2.0 * B[k].T @ G[k] @ B[k].T", "Mx = B[k].T @ G[k] @ B[k].T",
     [pins.pin_finite_differences, pins.pin_theta_zero]),
    ("cayley_vjp", "Mx = 2.0 * B[k].T @ G[k] @ B[k].T", "Mx = 2.0 * B[k] @ G[k] @ B[k]",
     [pins.pin_finite_differences, pins.pin_vjp_forms]),
    ("cayley_vjp", "out[k] = Mx[iu, ju] - Mx[ju, iu]", "out[k] = Mx[ju, iu] - Mx[iu, ju]",
     [pins.pin_finite_differences, pins.pin_theta_zero]),
    ("materialise", "W[:, s:s + r] @ P[j, :r, :r]", "W[:, s:s + r] @ P[j, :r, :r].T",
     [pins.pin_dense_block_diag, pins.pin_input_centric_equals_materialised]),
    ("materialise", "R[k, :r, :r] @ W[s:s + r, :]", "W[s:s + r, :]",
     [pins.pin_dense_block_diag, pins.pin_spectrum]),
    ("backward", "G_W[s:s + r, :] @ W0P[s:s + r, :].T", "W0P[s:s + r, :] @ G_W[s:s + r, :].T",
     [pins.pin_finite_differences, pins.pin_input_centric_equals_materialised]),
    ("backward", "g_x = g_y @ W", "g_x = g_y @ W0", [pins.pin_finite_differences, pins.pin_adjoint]),
    ("backward", "RW0[:, s:s + r].T @ G_W[:, s:s + r]", "RW0[:, s:s + r].T @ G_W[:, s:s + r] * 0.5",
     [pins.pin_finite_differences]),
    ("skew_from_theta", "if r < b:\n            Q[-1, r:, :] = 0.0", "if False:\n            Q[-1, r:, :] = 0.0",
     [pins.pin_dense_block_diag, pins.pin_padding_gradients]),
    # Cayley-Neumann series and its VJP
    ("cayley_neumann", "for _ in range(CNP_ORDER):", "for _ in range(CNP_ORDER - 1):",
     [pins.pin_cnp_golden, pins.pin_cnp_series_tail]),
    ("cayley_neumann", "out[k] = I + 2.0 * series", "out[k] = I + series",
     [pins.pin_cnp_golden, pins.pin_cnp_b3_closed_form]),
    ("cayley_neumann", "power = power @ q", "power = power @ q.T",
     [pins.pin_cnp_golden, pins.pin_cnp_series_tail]),
    ("cayley_neumann_vjp", "D += pw[i] @ G[n] @ pw[k - 1 - i]", "D += pw[i] @ G[n].T @ pw[k - 1 - i]",
     [pins.pin_cnp_finite_differences, pins.pin_cnp_vjp_frechet]),
    ("cayley_neumann_vjp", "Qt = Q[n].T", "Qt = Q[n]",
     [pins.pin_cnp_golden, pins.pin_cnp_vjp_frechet]),
    ("cayley_neumann_vjp", "D += pw[i] @ G[n] @ pw[k - 1 - i]", "D += pw[i] @ G[n] @ pw[i]",
     [pins.pin_cnp_finite_differences, pins.pin_cnp_vjp_frechet]),
    ("cayley_neumann_vjp", "D *= 2.0", "D *= 1.0", [pins.pin_cnp_golden, pins.pin_cnp_theta_zero]),
    # block-mixing permutations
    ("materialise_permuted", "W[np.ix_(np.asarray(perm_out), np.asarray(perm_in))] = M",
     "W = M[np.ix_(np.asarray(perm_out), np.asarray(perm_in))]",
     [pins.pin_perm_explicit_matrices]),
    ("fold_permutations", "np.ix_(np.asarray(perm_out), np.asarray(perm_in))",
     "np.ix_(np.argsort(perm_out), np.asarray(perm_in))",
     [pins.pin_perm_explicit_matrices, pins.pin_perm_finite_differences]),
    ("backward", "G_W = G_W[np.ix_(np.asarray(perm_out), np.asarray(perm_in))]", "G_W = G_W",
     [pins.pin_perm_finite_differences, pins.pin_perm_spectrum_and_routes]),
    ("forward_input_centric", "x = x[:, np.asarray(perm_in)]", "x = x[:, np.argsort(perm_in)]",
     [pins.pin_perm_spectrum_and_routes]),
    ("permutation_matrix", "M[np.arange(d), pi] = 1.0", "M[pi, np.arange(d)] = 1.0",
     [pins.pin_permutation_convention, pins.pin_perm_explicit_matrices]),
    # INT8 weights
    ("quantize_rows", "r = np.rint((W[i] / s[i]).astype(np.float32))",
     "r = np.floor((W[i] / s[i]).astype(np.float32) + 0.5)",
     [pins.pin_quantize_closed_forms]),
    ("quantize_rows", "s = (amax / np.float32(127.0)).astype(np.float32)",
     "s = (amax / np.float32(128.0)).astype(np.float32)",
     [pins.pin_quantize_closed_forms, pins.pin_quantize_error_bound]),
    ("quantize_rows", "amax = np.max(np.abs(W), axis=1).astype(np.float32)",
     "amax = np.full(W.shape[0], np.max(np.abs(W)), dtype=np.float32)",
     [pins.pin_quantize_closed_forms, pins.pin_quantize_error_bound]),
    ("dequantize_rows", "np.asarray(s, dtype=np.float64)[:, None] * np.asarray(q, dtype=np.float64)",
     "np.asarray(s, dtype=np.float64)[None, :1] * np.asarray(q, dtype=np.float64)",
     [pins.pin_quantize_closed_forms]),
]


def _install(monkeypatch, fname, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(O, fname)))
    assert old in src, (fname, old)
    ns = {}
    exec(compile(src.replace(old, new), f"<mutant {fname}>", "exec"), O.__dict__, ns)
    monkeypatch.setattr(O, fname, ns[fname])


@pytest.mark.parametrize("case", MUTATIONS, ids=lambda c: f"{c[0]}:{c[2][:30]}")
def test_planted_mistake_is_caught(monkeypatch, case):
    fname, old, new, catchers = case
    _install(monkeypatch, fname, old, new)
    caught = []
    for pin in catchers:
        try:
            pin()
        except (AssertionError, ValueError, IndexError, np_linalg_error()):
            caught.append(pin.__name__)
    assert caught, f"planted mistake in {fname} passed every pin {[p.__name__ for p in catchers]}"


def np_linalg_error():
    import numpy as np
    return np.linalg.LinAlgError
