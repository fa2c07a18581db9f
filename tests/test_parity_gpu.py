"""GPU parity: libpoetx (through the C ABI) against the float64 oracle on the
same seeded inputs.

Every case compares every output element (y, z, g_x and every generator
block of g_theta), the full-size workloads tile by tile as well, plus
properties that hold at any size.
"""
import math
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU too; every test here is gpu-marked
    pytest.skip("no GPU", allow_module_level=True)

import oracle.poetx_oracle as O  # noqa: E402
from orthogonal_equivalence_amd import poetx as P  # noqa: E402
from orthogonal_equivalence_amd.inputs import (CONFIGS, LayerSpec, make_layer,  # noqa: E402
                                               make_permutations, resized, round_to_dtype)
from tests import gpu_util as U  # noqa: E402
from tests.oracle_pins import load_closed_forms, load_cnp_closed_forms  # noqa: E402


def test_single_hip_runtime_loaded():
    """libpoetx must share torch's HIP runtime (exactly one libamdhip64)."""
    torch.zeros(1, device="cuda")
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(libs) == 1, libs
    assert any("libpoetx.so" in line for line in maps.splitlines())


# ------------------------------------------------------------- Cayley build
def _build(theta: np.ndarray, d: int, b: int, act=P.POETX_BF16):
    nb = -(-d // b)
    th = torch.from_numpy(np.ascontiguousarray(theta, dtype=np.float32)).cuda()
    f32 = torch.empty(nb, b, b, device="cuda")
    a = torch.empty(nb, b, b, device="cuda", dtype=torch.bfloat16) if act == P.POETX_BF16 else None
    ws = torch.empty(max(P.poetx_build_workspace_size(d, b), 1), device="cuda", dtype=torch.uint8)
    P.poetx_build_orthogonal(th, d, b, f32, a, act, ws)
    torch.cuda.synchronize()
    return f32, a


def test_build_golden_closed_forms():
    for name, b, theta, Rref in load_closed_forms():
        U.log(f"[build golden] {name} b={b}")
        f32, _ = _build(theta[None, :], b, b, P.POETX_F32)
        err = np.max(np.abs(U.host(f32)[0] - Rref))
        assert err <= 2e-7, (name, err)


@pytest.mark.parametrize("b,nb,sigma", [
    (2, 3, 0.5), (3, 2, 0.5), (8, 5, 0.3), (32, 8, 0.02), (48, 3, 0.1), (64, 4, 0.05),
    (96, 2, 0.05), (128, 3, 0.02), (256, 4, 0.01), (512, 2, 0.01), (1024, 1, 0.01),
    (256, 2, 0.2),
    # 48 blocks and more: b = 256 on the whole-block kernel, b = 512 as 2 x 2
    # pieces of 256 (Schur complement)
    (256, 48, 0.01), (512, 48, 0.01), (512, 50, 0.05),
    # the largest blocks the library takes (4096) and one below it
    (2048, 1, 0.004), (4096, 1, 0.002),
])
def test_build_matches_oracle(b, nb, sigma):
    U.log(f"[build] b={b} nb={nb} sigma={sigma}")
    rng = np.random.default_rng(b * 7 + nb)
    theta = (rng.standard_normal((nb, b * (b - 1) // 2)) * sigma).astype(np.float32).astype(np.float64)
    R_ref, _ = O.orthogonal_blocks(theta, b, nb * b)
    f32, act = _build(theta, nb * b, b)
    R = U.host(f32)
    err = np.max(np.abs(R - R_ref))
    U.log(f"    max abs err {err:.2e}")
    assert err <= 2e-5 * max(1.0, math.sqrt(b) / 8)
    I = np.eye(b)
    # float32 elimination: orthogonality defect grows like u b^1.5 (u = 2^-24)
    orth = max(np.linalg.norm(R[k].T @ R[k] - I) for k in range(nb))
    U.log(f"    ||R^T R - I||_F {orth:.2e}")
    assert orth <= 2.0 ** -24 * b ** 1.5 * 4
    # the bf16 copy is the RNE rounding of the float32 blocks
    a = act.float()
    ref = f32.to(torch.bfloat16).float()
    assert torch.equal(a, ref)


@pytest.mark.parametrize("b,nb", [(256, 3), (256, 48), (512, 2), (512, 48)])
def test_build_f32_only_matches_bf16_build(b, nb):
    """With act = float32 (no bf16 copy requested) each build form (panels,
    whole block, Schur pieces) writes the same float32 blocks as with the bf16
    copy, and they match the oracle."""
    U.log(f"[build f32] b={b} nb={nb}")
    rng = np.random.default_rng(31 * b + nb)
    theta = (rng.standard_normal((nb, b * (b - 1) // 2)) * 0.01).astype(np.float32).astype(np.float64)
    f32_only, none = _build(theta, nb * b, b, P.POETX_F32)
    assert none is None
    f32, _ = _build(theta, nb * b, b)
    assert torch.equal(f32_only, f32)
    R_ref, _ = O.orthogonal_blocks(theta, b, nb * b)
    assert np.max(np.abs(U.host(f32_only) - R_ref)) <= 2e-5 * max(1.0, math.sqrt(b) / 8)


@pytest.mark.parametrize("b,r,nfull", [(64, 24, 2), (128, 77, 2), (256, 24, 2), (256, 193, 2),
                                        (256, 193, 47), (512, 300, 47), (512, 200, 47),
                                        (512, 256, 47), (512, 257, 47)])
def test_build_padded_last_block(b, r, nfull):
    """b does not divide d: the last block is diag(Cayley(Q_r), I), with the
    valid part ending inside a 64-wide tile or at its first column. Three
    blocks run on the panel kernels (b = 64, 256) or the whole-block kernel
    (b = 128); 48 blocks on the whole-block kernel (b = 256) or as Schur
    pieces (b = 512, the valid part ending in either half, exactly at the
    half, or one row past it)."""
    d = b * nfull + r
    U.log(f"[build padded] b={b} d={d}")
    rng = np.random.default_rng(5 + b + r + nfull)
    sigma = 0.05 if b == 64 else 0.01
    theta = (rng.standard_normal((nfull + 1, b * (b - 1) // 2)) * sigma).astype(np.float32).astype(np.float64)
    R_ref, _ = O.orthogonal_blocks(theta, b, d)
    f32, act = _build(theta, d, b)
    R = U.host(f32)
    assert np.max(np.abs(R - R_ref)) <= 2e-5
    assert np.array_equal(R[-1, r:, r:], np.eye(b - r))
    assert np.all(R[-1, :r, r:] == 0) and np.all(R[-1, r:, :r] == 0)
    assert torch.equal(act.float(), f32.to(torch.bfloat16).float())


# ------------------------------------------------------ full layer, small
SMALL_CASES = [
    # name, d_in, d_out, b, tokens, dtype, sigma
    ("f32_tiles", 192, 320, 32, 200, "f32", 0.05),
    ("f32_b64_ragged_tokens", 256, 128, 64, 77, "f32", 0.05),
    ("f32_padded_blocks", 200, 136, 48, 130, "f32", 0.05),
    ("bf16_tiles", 512, 768, 128, 1000, "bf16", 0.02),
    ("bf16_b256", 512, 1024, 256, 300, "bf16", 0.01),
    ("bf16_b64_one_token", 256, 384, 64, 1, "bf16", 0.05),
    ("bf16_padded_blocks", 320, 200, 128, 257, "bf16", 0.02),
    ("bf16_b512", 1024, 512, 512, 129, "bf16", 0.01),
    # b = 512: the grams stream in four quadrant workgroups per block and
    # token range; the applies take the batched dense kernel at 1000 tokens
    # (several blocks, a ragged token tile) and the streaming slab
    # workgroups below 256 tokens (launches whose last group of 8 units is
    # partly padding)
    ("bf16_b512_blocks", 2048, 1536, 512, 1000, "bf16", 0.01),
    ("bf16_b512_padded_units", 1536, 1024, 512, 100, "bf16", 0.01),
    # one token: every streamed tile is ragged, every split but one empty
    ("bf16_b512_one_token", 512, 1024, 512, 1, "bf16", 0.01),
    ("bf16_b256_one_token", 768, 512, 256, 1, "bf16", 0.01),
    # b >= 512 on the batched dense kernel (ragged last 256-token tile), b =
    # 512 with both kernels in one layer (input side streamed: 544 tokens per
    # workgroup; output side dense), and b = 1024 below one 256-token tile
    # (generic batched GEMM)
    ("bf16_b1024_dense", 2048, 1024, 1024, 700, "bf16", 0.01),
    ("bf16_b512_stream_and_dense", 4096, 512, 512, 8300, "bf16", 0.01),
    ("bf16_b1024_few_tokens", 1024, 2048, 1024, 200, "bf16", 0.01),
    # b = 2048: two P blocks and one R block, batched dense block products
    ("bf16_b2048", 4096, 2048, 2048, 300, "bf16", 0.004),
    # b = 32 / 64 run as block-diagonal 128 x 128 super blocks on the b = 128
    # streaming kernels (128 divides d)
    ("bf16_b64_super", 384, 640, 64, 300, "bf16", 0.02),
    ("bf16_b32_super", 256, 384, 32, 200, "bf16", 0.05),
    # b = 256: the backward's gradient apply and gram share one pass over g_Y
    # (and over g_U); seven token splits, the last one ragged, and a padded
    # last group of units
    ("bf16_b256_splits", 768, 1280, 256, 2100, "bf16", 0.01),
    # whole 256-token panels: U (and g_Z) pass from the streaming applies to
    # the dense kernel in the tiled layout; b = 256 (R-apply in the dense
    # epilogue, one-pass backward), b = 128 (one-pass backward on the b = 128
    # kernel), b = 64 on super blocks, and b = 512 with the input side
    # streamed (544 tokens per workgroup) and the output side dense
    ("bf16_b256_tiled", 768, 1280, 256, 1536, "bf16", 0.01),
    ("bf16_b128_tiled", 512, 768, 128, 1024, "bf16", 0.02),
    ("bf16_b64_super_tiled", 384, 640, 64, 512, "bf16", 0.02),
    ("bf16_b512_stream_tiled", 4096, 512, 512, 8448, "bf16", 0.01),
]
SMALL_BY_NAME = {c[0]: c for c in SMALL_CASES}


@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: c[0])
def test_layer_small_full_compare(case):
    name, n, m, b, N, dt, sigma = case
    spec = LayerSpec(name, n, m, b, N, dt, sigma, seed=len(name))
    U.log(f"[layer] {name}: d_in={n} d_out={m} b={b} tokens={N} {dt}")
    L = make_layer(spec)
    ora = O.LayerOracle(L.W0, L.theta_R, L.theta_P, b, b)
    y_ref = ora.forward(L.x)
    gx_ref, gR_ref, gP_ref = ora.backward(L.g_y, L.x)
    lay, out = U.run_layer(L)
    U.check("R", U.host(lay.R_f32), ora.R, "f32")
    U.check("P", U.host(lay.P_f32), ora.P, "f32")
    U.check("y", U.host(out["y"]), y_ref, dt)
    _, z_ref, _ = O.forward_input_centric(L.x, L.W0, ora.R, ora.P, b, b)
    U.check("z", U.host(out["z"]), z_ref, dt)
    U.check("g_x", U.host(out["g_x"]), gx_ref, dt)
    U.check("g_theta_R", U.host(out["g_theta_R"]), gR_ref, dt)
    U.check("g_theta_P", U.host(out["g_theta_P"]), gP_ref, dt)


def test_tiny_config_exact_sizes():
    """The 256 x 256, b = 32, 64-token float32 workload, every element."""
    spec = CONFIGS["tiny_f32"][0]
    L = make_layer(spec)
    ora = O.LayerOracle(L.W0, L.theta_R, L.theta_P, spec.b, spec.b)
    y_ref = ora.forward(L.x)
    gx_ref, gR_ref, gP_ref = ora.backward(L.g_y, L.x)
    _, out = U.run_layer(L)
    U.check("y", U.host(out["y"]), y_ref, "f32")
    U.check("g_x", U.host(out["g_x"]), gx_ref, "f32")
    U.check("g_theta_R", U.host(out["g_theta_R"]), gR_ref, "f32")
    U.check("g_theta_P", U.host(out["g_theta_P"]), gP_ref, "f32")


def test_deterministic_bitwise():
    spec = LayerSpec("det", 512, 768, 128, 1000, "bf16", 0.02, seed=3)
    L = make_layer(spec)
    _, a = U.run_layer(L)
    _, c = U.run_layer(L)
    for k in ("y", "z", "g_x", "g_theta_R", "g_theta_P"):
        assert torch.equal(a[k], c[k]), k


def test_stage_events_with_null_entries():
    """Stage timing with NULL entries records only the given stages and leaves
    the results bit for bit unchanged (the benchmark times the dense product
    alone this way)."""
    from orthogonal_equivalence_amd.layer import PoetxLinear
    spec = LayerSpec("ev", 512, 1024, 256, 300, "bf16", 0.01, seed=4)
    L = make_layer(spec)
    _, ref = U.run_layer(L)
    lay = PoetxLinear(U.dev(L.W0, "bf16"), 256, 256, "bf16")
    lay.set_theta(torch.from_numpy(L.theta_R).float(), torch.from_numpy(L.theta_P).float())
    x, g_y = U.dev(L.x, "bf16"), U.dev(L.g_y, "bf16")
    e0, e1 = P.Event(), P.Event()
    lay.build()
    y, z = lay.forward(x, events=[None, None, e0.handle, e1.handle])
    g_x, gR, gP = lay.backward(g_y, x, z, events=[None] * 4 + [e0.handle, e1.handle])
    torch.cuda.synchronize()
    assert e0.elapsed_ms(e1) > 0.0
    for k, v in (("y", y), ("z", z), ("g_x", g_x), ("g_theta_R", gR), ("g_theta_P", gP)):
        assert torch.equal(v, ref[k]), k


def test_theta_zero_is_plain_linear():
    """theta = 0 gives R = P = I: y = x W0^T and g_x = g_y W0 (bf16 path)."""
    spec = LayerSpec("zero", 256, 512, 64, 130, "bf16", 0.0, seed=9)
    L = make_layer(spec)
    lay, out = U.run_layer(L)
    assert torch.equal(lay.R_f32, torch.eye(64, device="cuda").expand_as(lay.R_f32))
    U.check("y", U.host(out["y"]), L.x @ L.W0.T, "bf16")
    U.check("g_x", U.host(out["g_x"]), L.g_y @ L.W0, "bf16")


# ------------------------------------------------- full-size workloads
def _full_check(L, lay, out, map="cayley", perms=None, check_z=True):
    """Every output element of a full-size run against the oracle: y, z
    (the forward's saved product), g_x and every generator block of g_theta,
    each also tile by tile (256 x 256 pieces, or per block), so that a single
    wrong output tile fails. Plus a property that holds at any size: R is
    orthogonal per block, so ||y_t,k|| = ||z_t,k||."""
    s = L.spec
    b = s.b
    po, pi = perms if perms is not None else (None, None)
    ora = O.LayerOracle(L.W0, L.theta_R, L.theta_P, b, b, map=map, perm_out=po, perm_in=pi)
    U.check("R", U.host(lay.R_f32), ora.R, "f32")
    U.check("P", U.host(lay.P_f32), ora.P, "f32")
    U.check_tiles("y", U.host(out["y"]), ora.forward(L.x), s.dtype)
    if check_z and out.get("z") is not None and perms is None:
        _, z_ref, _ = O.forward_input_centric(L.x, L.W0, ora.R, ora.P, b, b)
        U.check_tiles("z", U.host(out["z"]), z_ref, s.dtype)
        del z_ref
    gx_ref, gR_ref, gP_ref = ora.backward(L.g_y, L.x)
    U.check_tiles("g_x", U.host(out["g_x"]), gx_ref, s.dtype)
    U.check_blocks("g_theta_R", U.host(out["g_theta_R"]), gR_ref, s.dtype)
    U.check_blocks("g_theta_P", U.host(out["g_theta_P"]), gP_ref, s.dtype)
    # (the series is orthogonal to O(|Q|^6), far below bf16 at these sizes)
    if out.get("z") is not None and perms is None:
        y = out["y"].float().view(s.tokens, -1, b)
        z = out["z"].float().view(s.tokens, -1, b)
        ny, nz = y.norm(dim=2), z.norm(dim=2)
        rel = ((ny - nz).norm() / nz.norm()).item()
        U.log(f"    block-norm preservation rel {rel:.2e}")
        assert rel <= 2e-2


def test_persistent_dense_ragged_full_compare():
    """4400 tokens, d_in = d_out = 4096, b = 256: 18 x 16 = 288 output tiles
    of 256 x 256 in both dense products, more than one per CU, so the
    persistent tile loop runs (several tiles per workgroup, the epilogue of
    one tile before the copies of the next), and the last row of tiles is
    ragged (shifted back inside M). Every element compared."""
    spec = LayerSpec("persistent_ragged", 4096, 4096, 256, 4400, "bf16", 0.01, seed=11)
    U.log(f"[layer] {spec.name}: d_in={spec.d_in} d_out={spec.d_out} b={spec.b} tokens={spec.tokens}")
    L = make_layer(spec)
    lay, out = U.run_layer(L)
    _full_check(L, lay, out)


@pytest.mark.parametrize("cfg", ["proj_1b", "mlp_up_8b", "sweep_b64", "sweep_b128", "sweep_b256",
                                 "sweep_b512", "sweep_b1024"])
def test_full_size_workload(cfg):
    for spec in CONFIGS[cfg]:
        U.log(f"[full] {cfg}/{spec.name}: {spec.d_out}x{spec.d_in} b={spec.b} tokens={spec.tokens}")
        L = make_layer(spec)
        lay, out = U.run_layer(L)
        _full_check(L, lay, out)
        del lay, out
        torch.cuda.empty_cache()


@pytest.mark.parametrize("layer", range(7))
def test_full_size_layer_set_8b(layer):
    spec = CONFIGS["layer_set_8b"][layer]
    U.log(f"[full] layer_set_8b/{spec.name}: {spec.d_out}x{spec.d_in} b={spec.b} tokens={spec.tokens}")
    L = make_layer(spec)
    lay, out = U.run_layer(L)
    _full_check(L, lay, out)
    del lay, out
    torch.cuda.empty_cache()


# ------------------------------------------- POET-Xmem: Z recomputed
@pytest.mark.parametrize("case", [SMALL_CASES[i] for i in (0, 2, 3, 5, 6, 9)] +
                         [SMALL_BY_NAME[k] for k in ("bf16_b256_tiled", "bf16_b128_tiled")],
                         ids=lambda c: c[0])
def test_recompute_z_small(case):
    """POETX_RECOMPUTE_Z: the oracle's results, and bit for bit those of the
    path that keeps Z (the same kernels recompute the same Z)."""
    name, n, m, b, N, dt, sigma = case
    spec = LayerSpec(name, n, m, b, N, dt, sigma, seed=len(name))
    U.log(f"[recompute-z] {name}: d_in={n} d_out={m} b={b} tokens={N} {dt}")
    L = make_layer(spec)
    ora = O.LayerOracle(L.W0, L.theta_R, L.theta_P, b, b)
    y_ref = ora.forward(L.x)
    gx_ref, gR_ref, gP_ref = ora.backward(L.g_y, L.x)
    _, mem = U.run_layer(L, recompute_z=True)
    assert mem["z"] is None
    U.check("y", U.host(mem["y"]), y_ref, dt)
    U.check("g_x", U.host(mem["g_x"]), gx_ref, dt)
    U.check("g_theta_R", U.host(mem["g_theta_R"]), gR_ref, dt)
    U.check("g_theta_P", U.host(mem["g_theta_P"]), gP_ref, dt)
    _, keep = U.run_layer(L)
    for k in ("y", "g_x", "g_theta_R", "g_theta_P"):
        assert torch.equal(mem[k], keep[k]), k


def test_recompute_z_full_size_mlp_up_8b():
    """The 8B MLP up-projection (14336 x 4096, b = 256, 8192 tokens) with Z
    recomputed: every element against the oracle, and equal to the stored-Z path."""
    spec = CONFIGS["mlp_up_8b"][0]
    U.log(f"[recompute-z full] {spec.name}: {spec.d_out}x{spec.d_in} b={spec.b} tokens={spec.tokens}")
    L = make_layer(spec)
    lay, mem = U.run_layer(L, recompute_z=True)
    _, keep = U.run_layer(L)
    for k in ("y", "g_x", "g_theta_R", "g_theta_P"):
        assert torch.equal(mem[k], keep[k]), k
    _full_check(L, lay, keep)
    del lay, mem, keep
    torch.cuda.empty_cache()


# ------------------------------- y kept in place of Z (POETX_SAVED_Y)
SAVED_Y_CASES = [SMALL_BY_NAME[k] for k in (
    "f32_tiles", "f32_padded_blocks", "bf16_tiles", "bf16_b256", "bf16_b64_one_token",
    "bf16_padded_blocks", "bf16_b512", "bf16_b256_one_token", "bf16_b1024_dense",
    "bf16_b32_super", "bf16_b256_splits", "bf16_b256_tiled", "bf16_b128_tiled")]


@pytest.mark.parametrize("case", SAVED_Y_CASES, ids=lambda c: c[0])
def test_saved_y_small(case):
    """POETX_SAVED_Y: the backward takes y, forms g_Y^T Y per R block and
    takes the factor R into the Cayley VJP (Z = Y R for orthogonal R). The
    oracle's gradients (formed from Z) to the usual tolerance; y and g_x bit
    for bit those of the stored-Z path (the same forward products, and g_Z =
    g_Y R does not involve Z). With 256 x 256 bf16 R blocks the forward writes
    no Z at all."""
    name, n, m, b, N, dt, sigma = case
    spec = LayerSpec(name, n, m, b, N, dt, sigma, seed=len(name) + 500)
    U.log(f"[saved-y] {name}: d_in={n} d_out={m} b={b} tokens={N} {dt}")
    L = make_layer(spec)
    ora = O.LayerOracle(L.W0, L.theta_R, L.theta_P, b, b)
    y_ref = ora.forward(L.x)
    gx_ref, gR_ref, gP_ref = ora.backward(L.g_y, L.x)
    _, sy = U.run_layer(L, saved_y=True)
    U.check("y", U.host(sy["y"]), y_ref, dt)
    U.check("g_x", U.host(sy["g_x"]), gx_ref, dt)
    U.check("g_theta_R", U.host(sy["g_theta_R"]), gR_ref, dt)
    U.check("g_theta_P", U.host(sy["g_theta_P"]), gP_ref, dt)
    _, keep = U.run_layer(L)
    for k in ("y", "g_x"):
        assert torch.equal(sy[k], keep[k]), k


def test_saved_y_full_size_mlp_up_8b():
    """The 8B MLP up-projection (14336 x 4096, b = 256, 8192 tokens) keeping
    y in place of Z: every element against the oracle; y and g_x equal to the
    stored-Z path."""
    spec = CONFIGS["mlp_up_8b"][0]
    U.log(f"[saved-y full] {spec.name}: {spec.d_out}x{spec.d_in} b={spec.b} tokens={spec.tokens}")
    L = make_layer(spec)
    lay, sy = U.run_layer(L, saved_y=True)
    _, keep = U.run_layer(L)
    for k in ("y", "g_x"):
        assert torch.equal(sy[k], keep[k]), k
    del keep
    _full_check(L, lay, sy)
    del lay, sy
    torch.cuda.empty_cache()


# ------------------- block sizes off the fast paths, and b_in != b_out
# R and P with different block sizes take separate builds and separate VJP
# launches; block sizes the streaming and whole-block kernels do not take
# run on the general GEMM and the panel build; ragged last blocks on either
# side. Every flag that changes the backward's route appears at least once.
ODD_BLOCK_CASES = [
    # name, d_in, d_out, b_in, b_out, tokens, dtype, sigma, options
    ("f32_b8_b16", 96, 128, 8, 16, 37, "f32", 0.05, {}),
    ("f32_b24_b12_ragged", 120, 76, 24, 12, 65, "f32", 0.05, {}),
    ("f32_b40_cnp", 200, 160, 40, 40, 50, "f32", 0.05, {"map": "cnp"}),
    # float32 activations at the larger blocks (general GEMM applies, the
    # whole-block and panel builds, the square float32 VJP products)
    ("f32_b128_b256", 512, 768, 128, 256, 300, "f32", 0.02, {}),
    ("f32_b256_saved_y", 512, 512, 256, 256, 257, "f32", 0.01, {"saved_y": True}),
    ("f32_b512_mem", 1024, 512, 512, 512, 100, "f32", 0.01, {"recompute_z": True}),
    ("bf16_b16_b40", 160, 200, 16, 40, 300, "bf16", 0.05, {}),
    ("bf16_b96_b80_ragged", 440, 328, 96, 80, 257, "bf16", 0.03, {}),
    ("bf16_b96_b160", 480, 640, 96, 160, 513, "bf16", 0.03, {}),
    ("bf16_b384", 768, 1152, 384, 384, 260, "bf16", 0.01, {}),
    ("bf16_b128_b256", 512, 1024, 128, 256, 1024, "bf16", 0.02, {}),
    ("bf16_b256_b128_saved_y", 768, 512, 256, 128, 700, "bf16", 0.02, {"saved_y": True}),
    ("bf16_b64_b256_mem", 512, 768, 64, 256, 512, "bf16", 0.02, {"recompute_z": True}),
    ("bf16_b256_b64_cnp", 512, 512, 256, 64, 300, "bf16", 0.02, {"map": "cnp"}),
    ("bf16_b24_cnp", 240, 168, 24, 24, 100, "bf16", 0.03, {"map": "cnp"}),
]


@pytest.mark.parametrize("case", ODD_BLOCK_CASES, ids=lambda c: c[0])
def test_layer_odd_and_unequal_blocks(case):
    from orthogonal_equivalence_amd.inputs import make_layer_blocks
    from orthogonal_equivalence_amd.layer import PoetxLinear
    name, n, m, b_in, b_out, N, dt, sigma, opts = case
    U.log(f"[odd blocks] {name}: d_in={n} d_out={m} b_in={b_in} b_out={b_out} tokens={N} {dt} "
          f"{opts}")
    L = make_layer_blocks(n, m, b_in, b_out, N, dt, sigma, seed=len(name) + 700)
    map_ = opts.get("map", "cayley")
    ora = O.LayerOracle(L["W0"], L["theta_R"], L["theta_P"], b_out, b_in, map=map_)
    y_ref = ora.forward(L["x"])
    gx_ref, gR_ref, gP_ref = ora.backward(L["g_y"], L["x"])
    lay = PoetxLinear(U.dev(L["W0"], dt), b_in, b_out, dt, **opts)
    lay.set_theta(torch.from_numpy(L["theta_R"]).float(), torch.from_numpy(L["theta_P"]).float())
    x, g_y = U.dev(L["x"], dt), U.dev(L["g_y"], dt)
    lay.build()
    y, z = lay.forward(x)
    g_x, gR, gP = lay.backward(g_y, x, z)
    torch.cuda.synchronize()
    U.check("R", U.host(lay.R_f32), ora.R, "f32")
    U.check("P", U.host(lay.P_f32), ora.P, "f32")
    U.check("y", U.host(y), y_ref, dt)
    U.check("g_x", U.host(g_x), gx_ref, dt)
    U.check("g_theta_R", U.host(gR), gR_ref, dt)
    U.check("g_theta_P", U.host(gP), gP_ref, dt)


# ----------------------------------------- Cayley-Neumann series (CNP)
def _build_cnp(theta: np.ndarray, d: int, b: int, act=P.POETX_BF16):
    nb = -(-d // b)
    th = torch.from_numpy(np.ascontiguousarray(theta, dtype=np.float32)).cuda()
    q = torch.empty(nb, b, b, device="cuda")
    f32 = torch.empty(nb, b, b, device="cuda")
    a = torch.empty(nb, b, b, device="cuda", dtype=torch.bfloat16) if act == P.POETX_BF16 else None
    ws = torch.empty(max(P.poetx_build_cnp_workspace_size(d, b), 1), device="cuda", dtype=torch.uint8)
    P.poetx_build_cnp(th, d, b, q, f32, a, act, ws)
    torch.cuda.synchronize()
    return q, f32, a


def test_cnp_build_golden():
    """Hand-derived series blocks (b = 4 pairs case; b = 2 is below the
    kernels' multiple-of-4 block size, so it is embedded in a b = 4 block
    whose other generators are zero)."""
    rows = [r for r in load_cnp_closed_forms() if r[0] == "R"]
    for kind, name, b, theta, vals, _ in rows:
        if b == 2:
            th4 = np.zeros(6)
            th4[0] = theta[0]          # (0, 1) coupling only
            ref = np.eye(4)
            ref[:2, :2] = vals
            b, theta, vals = 4, th4, ref
        U.log(f"[cnp golden] {name} b={b}")
        q, f32, _ = _build_cnp(theta[None, :], b, b, P.POETX_F32)
        scale = max(1.0, np.abs(vals).max())
        err = np.max(np.abs(U.host(f32)[0] - vals))
        assert err <= 4e-7 * scale, (name, err)
        assert np.array_equal(U.host(q)[0], O.skew_from_theta(theta[None, :].astype(np.float32), b)[0])


@pytest.mark.parametrize("b,nb,sigma", [
    (4, 3, 0.4), (8, 5, 0.3), (32, 8, 0.05), (48, 3, 0.1), (64, 4, 0.05), (128, 3, 0.02),
    (256, 4, 0.01), (512, 2, 0.01), (1024, 1, 0.005), (256, 3, 0.05),
])
def test_cnp_build_matches_oracle(b, nb, sigma):
    U.log(f"[cnp build] b={b} nb={nb} sigma={sigma}")
    rng = np.random.default_rng(b * 11 + nb)
    theta = (rng.standard_normal((nb, b * (b - 1) // 2)) * sigma).astype(np.float32).astype(np.float64)
    R_ref, Q_ref = O.orthogonal_blocks_cnp(theta, b, nb * b)
    q, f32, act = _build_cnp(theta, nb * b, b)
    assert np.array_equal(U.host(q), Q_ref)
    R = U.host(f32)
    err = np.max(np.abs(R - R_ref))
    U.log(f"    max abs err {err:.2e}")
    assert err <= 8e-6 * max(1.0, np.abs(R_ref).max())
    assert torch.equal(act.float(), f32.to(torch.bfloat16).float())


def test_cnp_build_padded_last_block():
    """b does not divide d: the last block is diag(series(Q_r), I)."""
    b, d = 48, 48 * 2 + 20
    rng = np.random.default_rng(6)
    theta = (rng.standard_normal((3, b * (b - 1) // 2)) * 0.1).astype(np.float32).astype(np.float64)
    R_ref, _ = O.orthogonal_blocks_cnp(theta, b, d)
    _, f32, _ = _build_cnp(theta, d, b)
    R = U.host(f32)
    assert np.max(np.abs(R - R_ref)) <= 2e-6
    assert np.array_equal(R[-1, 20:, 20:], np.eye(b - 20))
    assert np.all(R[-1, :20, 20:] == 0) and np.all(R[-1, 20:, :20] == 0)


# (the b = 64 bf16 case runs its grams as super blocks reduced in float32)
CNP_CASES = [SMALL_CASES[i] for i in (0, 1, 2, 3, 4, 6, 7)] + \
    [c for c in SMALL_CASES if c[0] == "bf16_b64_super"]


@pytest.mark.parametrize("case", CNP_CASES, ids=lambda c: c[0])
def test_cnp_layer_small_full_compare(case):
    name, n, m, b, N, dt, sigma = case
    spec = LayerSpec(name, n, m, b, N, dt, sigma, seed=len(name) + 100)
    U.log(f"[cnp layer] {name}: d_in={n} d_out={m} b={b} tokens={N} {dt}")
    L = make_layer(spec)
    ora = O.LayerOracle(L.W0, L.theta_R, L.theta_P, b, b, map="cnp")
    y_ref = ora.forward(L.x)
    gx_ref, gR_ref, gP_ref = ora.backward(L.g_y, L.x)
    lay, out = U.run_layer(L, map="cnp")
    U.check("R", U.host(lay.R_f32), ora.R, "f32")
    U.check("P", U.host(lay.P_f32), ora.P, "f32")
    U.check("y", U.host(out["y"]), y_ref, dt)
    U.check("g_x", U.host(out["g_x"]), gx_ref, dt)
    U.check("g_theta_R", U.host(out["g_theta_R"]), gR_ref, dt)
    U.check("g_theta_P", U.host(out["g_theta_P"]), gP_ref, dt)
    # Z recomputed in the backward: the same bits
    _, mem = U.run_layer(L, map="cnp", recompute_z=True)
    for k in ("y", "g_x", "g_theta_R", "g_theta_P"):
        assert torch.equal(mem[k], out[k]), k


def test_cnp_deterministic_bitwise():
    spec = LayerSpec("cnp_det", 512, 768, 128, 1000, "bf16", 0.02, seed=4)
    L = make_layer(spec)
    _, a = U.run_layer(L, map="cnp")
    _, c = U.run_layer(L, map="cnp")
    for k in ("y", "z", "g_x", "g_theta_R", "g_theta_P"):
        assert torch.equal(a[k], c[k]), k


def test_cnp_full_size_mlp_up_8b():
    """The 8B MLP up-projection (14336 x 4096, b = 256, 8192 tokens) with the
    series map: every element against the oracle."""
    spec = CONFIGS["mlp_up_8b"][0]
    U.log(f"[cnp full] {spec.name}: {spec.d_out}x{spec.d_in} b={spec.b} tokens={spec.tokens}")
    L = make_layer(spec)
    lay, out = U.run_layer(L, map="cnp")
    _full_check(L, lay, out, map="cnp")
    del lay, out
    torch.cuda.empty_cache()


# ------------------------------------------- block-mixing permutations
def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("dt,d_out,d_in", [
    ("bf16", 48, 4096), ("f32", 40, 1024), ("bf16", 9, 14336),
    ("bf16", 5, 40000), ("f32", 3, 20000),   # rows over 64 KB: the global-memory gather
])
def test_fold_weight_bit_exact(dt, d_out, d_in):
    U.log(f"[fold] {dt} {d_out}x{d_in}")
    rng = np.random.default_rng(d_out * 31 + d_in)
    W0 = round_to_dtype(rng.standard_normal((d_out, d_in)), dt)
    po, pi = rng.permutation(d_out), rng.permutation(d_in)
    act = P.POETX_BF16 if dt == "bf16" else P.POETX_F32
    Wd = U.dev(W0, dt)
    out = torch.empty_like(Wd)
    P.poetx_fold_weight(Wd, d_out, d_in, _i32(po), _i32(pi), act, out)
    torch.cuda.synchronize()
    assert np.array_equal(U.host(out), W0[np.ix_(po, pi)])


def test_fold_weight_out_of_range_entries_read_zero():
    """Entries outside [0, d) are bounds-checked in the kernel and read as zero."""
    rng = np.random.default_rng(3)
    d_out, d_in = 6, 64
    W0 = round_to_dtype(rng.standard_normal((d_out, d_in)), "bf16")
    po = np.array([5, 4, -1, 2, 6, 0])
    pi = rng.permutation(d_in)
    pi[[3, 17]] = [-7, d_in]
    out = torch.empty(d_out, d_in, device="cuda", dtype=torch.bfloat16)
    P.poetx_fold_weight(U.dev(W0, "bf16"), d_out, d_in, _i32(po), _i32(pi), P.POETX_BF16, out)
    torch.cuda.synchronize()
    got = U.host(out)
    ref = np.zeros((d_out, d_in))
    for i in range(d_out):
        for j in range(d_in):
            if 0 <= po[i] < d_out and 0 <= pi[j] < d_in:
                ref[i, j] = W0[po[i], pi[j]]
    assert np.array_equal(got, ref)


PERM_CASES = [
    # name, d_in, d_out, b, tokens, dtype, sigma, map
    ("perm_f32_tiles", 192, 320, 32, 200, "f32", 0.05, "cayley"),
    ("perm_f32_padded_cnp", 200, 136, 48, 130, "f32", 0.05, "cnp"),
    ("perm_bf16_b128", 512, 768, 128, 1000, "bf16", 0.02, "cayley"),
    ("perm_bf16_b256_cnp", 512, 1024, 256, 300, "bf16", 0.01, "cnp"),
    ("perm_bf16_padded", 320, 200, 128, 257, "bf16", 0.02, "cayley"),
    ("perm_bf16_b512", 1024, 1536, 512, 300, "bf16", 0.01, "cayley"),
    ("perm_bf16_b64_super", 384, 640, 64, 300, "bf16", 0.02, "cayley"),
]


@pytest.mark.parametrize("case", PERM_CASES, ids=lambda c: c[0])
def test_perm_layer_small_full_compare(case):
    name, n, m, b, N, dt, sigma, map_ = case
    spec = LayerSpec(name, n, m, b, N, dt, sigma, seed=len(name) + 200)
    U.log(f"[perm layer] {name}: d_in={n} d_out={m} b={b} tokens={N} {dt} {map_}")
    L = make_layer(spec)
    po, pi = make_permutations(spec)
    ora = O.LayerOracle(L.W0, L.theta_R, L.theta_P, b, b, map=map_, perm_out=po, perm_in=pi)
    y_ref = ora.forward(L.x)
    gx_ref, gR_ref, gP_ref = ora.backward(L.g_y, L.x)
    lay, out = U.run_layer(L, map=map_, perms=(po, pi))
    assert np.array_equal(U.host(lay.W0), L.W0[np.ix_(po, pi)])
    U.check("y", U.host(out["y"]), y_ref, dt)
    U.check("g_x", U.host(out["g_x"]), gx_ref, dt)
    U.check("g_theta_R", U.host(out["g_theta_R"]), gR_ref, dt)
    U.check("g_theta_P", U.host(out["g_theta_P"]), gP_ref, dt)
    # Z recomputed from the gathered x: the same bits
    _, mem = U.run_layer(L, map=map_, perms=(po, pi), recompute_z=True)
    for k in ("y", "g_x", "g_theta_R", "g_theta_P"):
        assert torch.equal(mem[k], out[k]), k


def test_perm_identity_maps_bitwise():
    """Identity index maps: every output bit for bit that of the layer
    without permutations (gathers by the identity copy exactly)."""
    spec = LayerSpec("perm_id", 512, 768, 128, 1000, "bf16", 0.02, seed=21)
    L = make_layer(spec)
    _, a = U.run_layer(L)
    _, c = U.run_layer(L, perms=(np.arange(768), np.arange(512)))
    for k in ("y", "z", "g_x", "g_theta_R", "g_theta_P"):
        assert torch.equal(a[k], c[k]), k


def test_perm_full_size_mlp_up_8b():
    """The 8B MLP up-projection (14336 x 4096, b = 256, 8192 tokens) with
    random block-mixing permutations: every element against the oracle."""
    spec = CONFIGS["mlp_up_8b"][0]
    U.log(f"[perm full] {spec.name}: {spec.d_out}x{spec.d_in} b={spec.b} tokens={spec.tokens}")
    L = make_layer(spec)
    po, pi = make_permutations(spec)
    lay, out = U.run_layer(L, perms=(po, pi))
    _full_check(L, lay, out, perms=(po, pi))
    del lay, out
    torch.cuda.empty_cache()


# ------------------------------------------- INT8 frozen weight (POET-XQ)
@pytest.mark.parametrize("dt,d_out,d_in", [("bf16", 200, 512), ("f32", 64, 136), ("bf16", 14336, 4096)])
def test_quantize_weight_bit_exact(dt, d_out, d_in):
    """Codes and scales equal the oracle's (decided in float32 on both sides),
    including a zero row and rows with exact ties."""
    U.log(f"[quantize] {dt} {d_out}x{d_in}")
    rng = np.random.default_rng(d_out + d_in)
    W = rng.standard_normal((d_out, d_in)) * rng.uniform(0.01, 2.0, (d_out, 1))
    W[1] = 0.0
    u = 2.0 ** -7
    W[2] = u * np.resize(np.array([2.5, 3.5, -2.5, -0.5, 127.0, 1.5]), d_in)
    W = round_to_dtype(W, dt)
    act = P.POETX_BF16 if dt == "bf16" else P.POETX_F32
    q = torch.empty(d_out, d_in, device="cuda", dtype=torch.int8)
    sc = torch.empty(d_out, device="cuda", dtype=torch.float32)
    P.poetx_quantize_weight(U.dev(W, dt), d_out, d_in, act, q, sc)
    torch.cuda.synchronize()
    q_ref, s_ref = O.quantize_rows(W)
    assert np.array_equal(sc.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def _int8_reference_inputs(L):
    """The layer inputs with W0 replaced by diag(s) q of the oracle's codes."""
    import dataclasses
    q, s = O.quantize_rows(L.W0)
    return dataclasses.replace(L, W0=O.dequantize_rows(q, s))


INT8_CASES = [
    # name, d_in, d_out, b, tokens, dtype, sigma, map, permute, recompute
    ("q8_f32_tiles", 192, 320, 32, 200, "f32", 0.05, "cayley", False, False),
    ("q8_bf16_b128", 512, 768, 128, 1000, "bf16", 0.02, "cayley", False, False),
    ("q8_bf16_padded_cnp", 320, 200, 128, 257, "bf16", 0.02, "cnp", False, False),
    ("q8_bf16_b256_perm_mem", 512, 1024, 256, 300, "bf16", 0.01, "cayley", True, True),
    ("q8_bf16_b512_mem", 1024, 1536, 512, 200, "bf16", 0.01, "cayley", False, True),
    ("q8_bf16_b64_super", 384, 640, 64, 300, "bf16", 0.02, "cayley", False, False),
    # enough tokens that the codes are widened in chunks (at 16384 tokens
    # 2048 weight rows forward, 1024 columns backward): forward 2048 + 2048 +
    # 512 rows with the fused R-apply, backward 1024 + 1024 + 256 columns;
    # then b = 128 (separate R-apply) with Z recomputed, where the forward's
    # last chunk takes the 128-row remainder (2048 + 2176) and the backward's
    # too (1024 + 1152)
    ("q8_bf16_b256_chunks", 2304, 4608, 256, 16384, "bf16", 0.01, "cayley", False, False),
    ("q8_bf16_b128_chunks_mem", 2176, 4224, 128, 16384, "bf16", 0.02, "cayley", False, True),
]


@pytest.mark.parametrize("case", INT8_CASES, ids=lambda c: c[0])
def test_int8_layer_small_full_compare(case):
    name, n, m, b, N, dt, sigma, map_, permute, mem = case
    spec = LayerSpec(name, n, m, b, N, dt, sigma, seed=len(name) + 300)
    U.log(f"[int8 layer] {name}: d_in={n} d_out={m} b={b} tokens={N} {dt} {map_} "
          f"perm={permute} recompute={mem}")
    L = make_layer(spec)
    po, pi = make_permutations(spec) if permute else (None, None)
    Lq = _int8_reference_inputs(L)
    ora = O.LayerOracle(Lq.W0, L.theta_R, L.theta_P, b, b, map=map_, perm_out=po, perm_in=pi)
    y_ref = ora.forward(L.x)
    gx_ref, gR_ref, gP_ref = ora.backward(L.g_y, L.x)
    from orthogonal_equivalence_amd.layer import PoetxLinear
    lay = PoetxLinear(U.dev(L.W0, dt), b, b, dt, map=map_, perm_out=po, perm_in=pi, int8=True,
                      recompute_z=mem)
    assert lay.W0.dtype == torch.int8
    lay.set_theta(torch.from_numpy(L.theta_R).float(), torch.from_numpy(L.theta_P).float())
    x, g_y = U.dev(L.x, dt), U.dev(L.g_y, dt)
    lay.build()
    y, z = lay.forward(x)
    g_x, gR, gP = lay.backward(g_y, x, z)
    torch.cuda.synchronize()
    U.check("y", U.host(y), y_ref, dt)
    U.check("g_x", U.host(g_x), gx_ref, dt)
    U.check("g_theta_R", U.host(gR), gR_ref, dt)
    U.check("g_theta_P", U.host(gP), gP_ref, dt)


def test_int8_full_size_mlp_up_8b():
    """The 8B MLP up-projection with an INT8 weight: oracle checks
    against the dequantised weight, every element."""
    spec = CONFIGS["mlp_up_8b"][0]
    U.log(f"[int8 full] {spec.name}: {spec.d_out}x{spec.d_in} b={spec.b} tokens={spec.tokens}")
    L = make_layer(spec)
    from orthogonal_equivalence_amd.layer import PoetxLinear
    lay = PoetxLinear(U.dev(L.W0, spec.dtype), spec.b, spec.b, spec.dtype, int8=True)
    lay.set_theta(torch.from_numpy(L.theta_R).float(), torch.from_numpy(L.theta_P).float())
    x, g_y = U.dev(L.x, spec.dtype), U.dev(L.g_y, spec.dtype)
    lay.build()
    y, z = lay.forward(x)
    g_x, gR, gP = lay.backward(g_y, x, z)
    torch.cuda.synchronize()
    out = dict(y=y, z=None, g_x=g_x, g_theta_R=gR, g_theta_P=gP)
    _full_check(_int8_reference_inputs(L), lay, out, check_z=False)
    del lay, out, y, z, g_x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("case", [c for c in INT8_CASES
                                  if c[7] == "cayley" and not c[8] and not c[9]],
                         ids=lambda c: c[0])
def test_saved_y_int8(case):
    """POETX_SAVED_Y with an INT8 weight: Y already carries the row scales,
    so the R gram g_Y^T Y is taken without column scaling."""
    name, n, m, b, N, dt, sigma, map_, _, _ = case
    spec = LayerSpec(name, n, m, b, N, dt, sigma, seed=len(name) + 600)
    U.log(f"[saved-y int8] {name}: d_in={n} d_out={m} b={b} tokens={N} {dt}")
    L = make_layer(spec)
    ora = O.LayerOracle(_int8_reference_inputs(L).W0, L.theta_R, L.theta_P, b, b)
    y_ref = ora.forward(L.x)
    gx_ref, gR_ref, gP_ref = ora.backward(L.g_y, L.x)
    _, sy = U.run_layer(L, saved_y=True, int8=True)
    U.check("y", U.host(sy["y"]), y_ref, dt)
    U.check("g_x", U.host(sy["g_x"]), gx_ref, dt)
    U.check("g_theta_R", U.host(sy["g_theta_R"]), gR_ref, dt)
    U.check("g_theta_P", U.host(sy["g_theta_P"]), gP_ref, dt)


# ------------------------------------------- the step captured in a HIP graph
@pytest.mark.parametrize("case,kw", [
    (("bf16_b256_tiled", 768, 1280, 256, 1536), {}),
    (("bf16_b128_int8", 512, 768, 128, 1000), {"int8": True}),
    (("bf16_b256_mem", 512, 1024, 256, 300), {"recompute_z": True}),
    (("bf16_b256_saved_y", 768, 1280, 256, 1536), {"saved_y": True}),
], ids=lambda c: c[0] if isinstance(c, tuple) else "-".join(c) or "plain")
def test_step_in_hip_graph(case, kw):
    """Build, forward and backward captured in one HIP graph (the library
    allocates nothing and records no memset inside a call) and replayed three
    times, with eager steps and synchronisations between the replays: every
    replay's outputs bit for bit those of the eager step."""
    from orthogonal_equivalence_amd.layer import PoetxLinear
    name, n, m, b, N = case
    spec = LayerSpec(name, n, m, b, N, "bf16", 0.01, seed=len(name) + 600)
    U.log(f"[hip graph] {name}: d_in={n} d_out={m} b={b} tokens={N} {kw}")
    L = make_layer(spec)
    lay = PoetxLinear(U.dev(L.W0, "bf16"), b, b, "bf16", **kw)
    lay.set_theta(torch.from_numpy(L.theta_R).float(), torch.from_numpy(L.theta_P).float())
    x, g_y = U.dev(L.x, "bf16"), U.dev(L.g_y, "bf16")
    y = torch.empty(N, m, dtype=torch.bfloat16, device="cuda")
    z = None if kw.get("recompute_z") or kw.get("saved_y") else torch.empty_like(y)
    saved = y if kw.get("saved_y") else z  # what the backward takes
    g_x = torch.empty(N, n, dtype=torch.bfloat16, device="cuda")
    gR, gP = torch.empty_like(lay.theta_R), torch.empty_like(lay.theta_P)
    side = torch.cuda.Stream()

    def step(stream):
        lay.build(stream)
        lay.forward(x, y, z, stream=stream)
        lay.backward(g_y, x, saved, g_x, gR, gP, stream=stream)

    def outputs():
        return [t.clone() for t in (y, g_x, gR, gP) + ((z,) if z is not None else ())]

    with torch.cuda.stream(side):
        step(side)  # workspaces allocated outside the capture
    torch.cuda.synchronize()
    ref = outputs()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(side)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (y, g_x, gR, gP):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, c in zip(ref, outputs()):
            assert torch.equal(a, c), rep
        step(torch.cuda.current_stream())  # eager work between the replays
        torch.cuda.synchronize()
        for a, c in zip(ref, outputs()):
            assert torch.equal(a, c), rep
