"""bench.py on the CPU: the one-GPU guard and the algorithmic work model."""
import importlib.util
import os
import subprocess
import sys

from orthogonal_equivalence_amd.inputs import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_layer_work_counts_every_product_of_the_step():
    """Flops of one step, summed product by product: S2, S4, B1, B2, B4, B5
    are token x block products (2 N d b each), S3 and B3 the dense W0
    products (2 N m n each), and per block the Cayley build (2 b^3) and VJP
    (two products, 4 b^3)."""
    b_mod = _bench_module()
    s = CONFIGS["mlp_up_8b"][0]
    N, n, m, b = s.tokens, s.d_in, s.d_out, s.b
    products = [2 * N * n * b,      # S2  U = X P^T
                2 * N * m * n,      # S3  Z = U W0^T
                2 * N * m * b,      # S4  Y = Z R^T
                2 * N * m * b,      # B1  g_Z = g_Y R
                2 * N * m * b,      # B2  G_R = g_Y^T Z
                2 * N * m * n,      # B3  g_U = g_Z W0
                2 * N * n * b,      # B4  G_P = g_U^T X
                2 * N * n * b]      # B5  g_X = g_U P
    nblocks = (m + n) // b
    products += [nblocks * 2 * b ** 3, nblocks * 4 * b ** 3]
    flops, nbytes = b_mod.layer_work(s)
    assert flops == sum(products)
    # bytes: at least every activation tensor the step must read or write once
    es = 2
    assert nbytes >= es * (N * n + N * m + N * m + N * n)


def test_layer_work_without_z_drops_one_activation_write():
    """With y kept in Z's place the forward writes one [tokens, d_out] tensor
    fewer; the flops are the same (the R gram's factor R moves into the VJP's
    first product, which has the same size)."""
    b_mod = _bench_module()
    s = CONFIGS["mlp_up_8b"][0]
    f0, b0 = b_mod.layer_work(s)
    f1, b1 = b_mod.layer_work(s, saved_y=True)
    assert f1 == f0
    assert b0 - b1 == 2 * s.tokens * s.d_out
