"""The oracle against what the method and mathematics fix (CPU only)."""
import numpy as np
import pytest

import oracle.poetx_oracle as O
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_spectrum_1b_projection_size():
    """Spectrum preservation at the 1B-class projection size (2048 x 2048,
    b = 256, theta ~ N(0, 0.01^2)): the pages' spectrum-preservation claim."""
    from orthogonal_equivalence_amd.inputs import CONFIGS, make_layer, resized
    spec = resized(CONFIGS["proj_1b"][0], tokens=1)
    L = make_layer(spec)
    ora = O.LayerOracle(L.W0, L.theta_R, L.theta_P, spec.b, spec.b)
    R = ora.R
    I = np.eye(spec.b)
    assert max(np.linalg.norm(R[k].T @ R[k] - I) for k in range(len(R))) <= 1e-10
    s = np.linalg.svd(ora.W, compute_uv=False)
    s0 = np.linalg.svd(L.W0, compute_uv=False)
    assert np.max(np.abs(s - s0)) / s0[0] <= 1e-9


def test_tiny_config_orthogonality_and_routes():
    from orthogonal_equivalence_amd.inputs import CONFIGS, make_layer
    spec = CONFIGS["tiny_f32"][0]
    L = make_layer(spec)
    ora = O.LayerOracle(L.W0, L.theta_R, L.theta_P, spec.b, spec.b)
    I = np.eye(spec.b)
    for blocks in (ora.R, ora.P):
        assert max(np.linalg.norm(q.T @ q - I) for q in blocks) <= 1e-10
    y = ora.forward(L.x)
    y2, _, _ = O.forward_input_centric(L.x, L.W0, ora.R, ora.P, spec.b, spec.b)
    assert np.max(np.abs(y - y2)) <= 1e-12 * np.abs(y).max()
