"""The C ABI without a GPU: symbols, sizes and every host-detectable error.

Argument validation runs before any HIP call, so these run on the CPU.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "poetx.h")

P = pytest.importorskip("orthogonal_equivalence_amd.poetx",
                        reason="libpoetx.so not built (run the build first)")

ALIGNED = 1 << 20  # a fake 16-byte aligned address; validation never dereferences it


@pytest.fixture(autouse=True)
def _cpu_only():
    """Every call here is meant to stop in host validation; on a machine with a
    visible GPU a call that got past it would launch on fake addresses, so
    these tests run only where no GPU is visible."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-validation tests use fake device addresses; run them without a GPU")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(poetx_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(P.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(P.EXPORTS)


def test_version_and_strings():
    assert P.poetx_abi_version() == P.POETX_ABI_VERSION == 7
    for s in range(8):
        assert P.status_string(s) and P.status_string(s) != "unknown status"
    assert P.status_string(99) == "unknown status"


@pytest.mark.parametrize("d,b", [(256, 32), (14336, 256), (4096, 512), (10, 4), (7, 7), (4096, 1)])
def test_theta_count(d, b):
    nb = -(-d // b)
    assert P.poetx_num_blocks(d, b) == nb
    assert P.poetx_theta_count(d, b) == nb * b * (b - 1) // 2


def test_sizes_of_invalid_inputs_are_zero():
    assert P.poetx_theta_count(0, 4) == 0 and P.poetx_theta_count(4, 0) == 0
    assert P.poetx_build_workspace_size(4, 8) == 0  # b > d
    assert P.poetx_build_workspace_size(8192, 8192) == 0  # b > max block
    assert P.poetx_fwd_workspace_size(P.make_desc(0, 64, 64, 8, 8, P.POETX_BF16)) == 0
    assert P.poetx_bwd_workspace_size(P.make_desc(16, 64, 64, 8, 8, 5)) == 0


def test_workspace_sizes_positive():
    d = P.make_desc(8192, 4096, 14336, 256, 256, P.POETX_BF16)
    assert P.poetx_fwd_workspace_size(d) >= 8192 * 4096 * 2
    assert P.poetx_bwd_workspace_size(d) >= 8192 * (4096 + 14336) * 2
    assert P.poetx_build_workspace_size(14336 + 4096, 256) > 0


def _fwd(desc, **over):
    args = dict(x=ALIGNED, W0=ALIGNED * 2, R=ALIGNED * 3, P=ALIGNED * 4, y=ALIGNED * 64,
                z=ALIGNED * 128, ws=ALIGNED * 256, ws_bytes=1 << 40)
    args.update(over)
    d = desc
    return P._lib.poetx_linear_fwd(ctypes.byref(d), args["x"], args["W0"], args["R"], args["P"],
                                   args["y"], args["z"], args["ws"], args["ws_bytes"], None)


def _bwd(desc, **over):
    a = dict(g_y=ALIGNED, x=ALIGNED * 2, W0=ALIGNED * 3, Rf=ALIGNED * 4, Pf=ALIGNED * 5,
             Ra=ALIGNED * 6, Pa=ALIGNED * 7, z=ALIGNED * 8, g_x=ALIGNED * 64, gR=ALIGNED * 128,
             gP=ALIGNED * 192, ws=ALIGNED * 256, ws_bytes=1 << 40)
    a.update(over)
    return P._lib.poetx_linear_bwd(ctypes.byref(desc), a["g_y"], a["x"], a["W0"], a["Rf"], a["Pf"],
                                   a["Ra"], a["Pa"], a["z"], a["g_x"], a["gR"], a["gP"], a["ws"],
                                   a["ws_bytes"], None)


SMALL = dict(tokens=16, d_in=64, d_out=64, b_in=8, b_out=8, act=P.POETX_BF16)


def desc(**over):
    k = dict(SMALL)
    k.update(over)
    return P.make_desc(k["tokens"], k["d_in"], k["d_out"], k["b_in"], k["b_out"], k["act"],
                       flags=k.get("flags", 0), perm_in=k.get("perm_in"),
                       perm_out=k.get("perm_out"), w_scale=k.get("w_scale"))


@pytest.mark.parametrize("call", [_fwd, _bwd])
def test_null_pointers(call):
    keys = ["x", "W0", "R", "P", "y", "z"] if call is _fwd else \
        ["g_y", "x", "W0", "Rf", "Pf", "Ra", "Pa", "z", "g_x", "gR", "gP"]
    for k in keys:
        assert call(desc(), **{k: None}) == P.POETX_ERR_NULL, k
    assert P._lib.poetx_linear_fwd(None, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED,
                                   ALIGNED, 1, None) == P.POETX_ERR_NULL


@pytest.mark.parametrize("call", [_fwd, _bwd])
@pytest.mark.parametrize("bad", [
    dict(tokens=0), dict(d_in=0), dict(d_out=-8), dict(b_in=0), dict(b_out=0),
    dict(b_in=128), dict(b_out=8192, d_out=16384), dict(tokens=1 << 32),
])
def test_bad_shapes(call, bad):
    assert call(desc(**bad)) == P.POETX_ERR_SHAPE


@pytest.mark.parametrize("call", [_fwd, _bwd])
def test_bad_dtype(call):
    assert call(desc(act=2)) == P.POETX_ERR_DTYPE
    assert call(desc(act=-1)) == P.POETX_ERR_DTYPE


@pytest.mark.parametrize("call", [_fwd, _bwd])
@pytest.mark.parametrize("bad", [dict(d_in=60), dict(d_out=36), dict(b_in=12, d_in=48),
                                 dict(b_out=4)])
def test_alignment_of_sizes(call, bad):
    assert call(desc(**bad)) == P.POETX_ERR_ALIGN


def test_fp32_allows_multiples_of_four():
    d = desc(act=P.POETX_F32, d_in=60, b_in=12, b_out=4)
    assert P.poetx_fwd_workspace_size(d) > 0


@pytest.mark.parametrize("call", [_fwd, _bwd])
def test_misaligned_pointers(call):
    key = "x"
    assert call(desc(), **{key: ALIGNED + 2}) == P.POETX_ERR_ALIGN


@pytest.mark.parametrize("call", [_fwd, _bwd])
def test_workspace_too_small(call):
    d = desc()
    need = (P.poetx_fwd_workspace_size if call is _fwd else P.poetx_bwd_workspace_size)(d)
    assert call(d, ws_bytes=need - 1) == P.POETX_ERR_WORKSPACE
    assert call(d, ws=None) == P.POETX_ERR_WORKSPACE


def test_aliasing_is_rejected():
    d = desc()
    assert _fwd(d, y=ALIGNED) == P.POETX_ERR_ALIAS           # y on top of x
    assert _fwd(d, z=ALIGNED * 64) == P.POETX_ERR_ALIAS      # z on top of y
    assert _bwd(d, g_x=ALIGNED * 8) == P.POETX_ERR_ALIAS     # g_x on top of z
    assert _bwd(d, gR=ALIGNED * 256) == P.POETX_ERR_ALIAS    # g_theta_R inside the workspace


def test_workspace_is_a_written_buffer_for_alias_checks():
    """The kernels write U, Z, g_Z, g_U and the gram partials into the
    workspace, so a workspace on top of any input is an alias too."""
    d = desc()
    assert _fwd(d, ws=ALIGNED) == P.POETX_ERR_ALIAS            # on top of x
    assert _fwd(d, ws=ALIGNED * 2) == P.POETX_ERR_ALIAS        # on top of W0
    assert _fwd(d, ws=ALIGNED * 4) == P.POETX_ERR_ALIAS        # on top of P_act
    assert _fwd(d, ws=ALIGNED * 64) == P.POETX_ERR_ALIAS       # on top of y
    assert _bwd(d, ws=ALIGNED) == P.POETX_ERR_ALIAS            # on top of g_y
    assert _bwd(d, ws=ALIGNED * 2) == P.POETX_ERR_ALIAS        # on top of x
    assert _bwd(d, ws=ALIGNED * 5) == P.POETX_ERR_ALIAS        # on top of P_f32
    assert _bwd(d, ws=ALIGNED * 8) == P.POETX_ERR_ALIAS        # on top of z
    assert _bwd(d, ws=ALIGNED * 64) == P.POETX_ERR_ALIAS       # on top of g_x
    dp = desc(**PERMS)
    assert _fwd(dp, ws=ALIGNED * 300) == P.POETX_ERR_ALIAS     # on top of perm_in
    assert _bwd(dp, ws=ALIGNED * 301) == P.POETX_ERR_ALIAS     # on top of perm_out
    dq = desc(w_scale=ALIGNED * 500)
    assert _fwd(dq, ws=ALIGNED * 500) == P.POETX_ERR_ALIAS     # on top of the row scales


def test_events_without_array_rejected():
    d = desc()
    d.n_events = 4
    assert _fwd(d) == P.POETX_ERR_NULL


def _build(theta, d, b, f32, act_ptr, act, ws, ws_bytes):
    return P._lib.poetx_build_orthogonal(theta, d, b, f32, act_ptr, act, ws, ws_bytes, None)


def test_build_errors():
    ok = dict(theta=ALIGNED, d=64, b=8, f32=ALIGNED * 2, act_ptr=ALIGNED * 3, act=P.POETX_BF16,
              ws=ALIGNED * 4, ws_bytes=1 << 30)

    def call(**over):
        a = dict(ok)
        a.update(over)
        return _build(a["theta"], a["d"], a["b"], a["f32"], a["act_ptr"], a["act"], a["ws"],
                      a["ws_bytes"])

    assert call(theta=None) == P.POETX_ERR_NULL
    assert call(f32=None) == P.POETX_ERR_NULL
    assert call(act_ptr=None) == P.POETX_ERR_NULL
    assert call(act=7) == P.POETX_ERR_DTYPE
    assert call(d=0) == P.POETX_ERR_SHAPE
    assert call(b=0) == P.POETX_ERR_SHAPE
    assert call(b=128) == P.POETX_ERR_SHAPE               # b > d
    assert call(d=1 << 20, b=8192) == P.POETX_ERR_SHAPE   # b above the maximum
    assert call(f32=ALIGNED * 2 + 4) == P.POETX_ERR_ALIGN
    assert call(ws_bytes=16) == P.POETX_ERR_WORKSPACE
    assert call(ws=None) == P.POETX_ERR_WORKSPACE
    assert call(f32=ALIGNED) == P.POETX_ERR_ALIAS          # output on top of theta
    assert call(act_ptr=ALIGNED * 4) == P.POETX_ERR_ALIAS  # act copy inside the workspace
    assert call(ws=ALIGNED) == P.POETX_ERR_ALIAS           # workspace on top of theta


# -- POETX_RECOMPUTE_Z (POET-Xmem: Z is not kept by the forward) --------------

def test_unknown_flags_and_reserved_rejected():
    for call in (_fwd, _bwd):
        assert call(desc(flags=8)) == P.POETX_ERR_SHAPE
        assert call(desc(flags=16 | P.POETX_CAYLEY_NEUMANN)) == P.POETX_ERR_SHAPE
        assert call(desc(flags=-1)) == P.POETX_ERR_SHAPE
        d = desc()
        d.reserved = 1
        assert call(d) == P.POETX_ERR_SHAPE
    d = desc()
    d.reserved = 3
    assert P.poetx_fwd_workspace_size(d) == 0 and P.poetx_bwd_workspace_size(d) == 0


def test_recompute_z_takes_null_z_and_only_null():
    d = desc(flags=P.POETX_RECOMPUTE_Z)
    assert _fwd(d) == P.POETX_ERR_NULL          # a z_save buffer is not taken
    assert _bwd(d) == P.POETX_ERR_NULL          # nor a z_saved one
    assert _fwd(desc(), z=None) == P.POETX_ERR_NULL   # without the flag Z is required
    # with the flag and z NULL, only the (fake) workspace size stands between the
    # call and a launch: check it with a workspace that is one byte short
    need = P.poetx_fwd_workspace_size(d)
    assert _fwd(d, z=None, ws_bytes=need - 1) == P.POETX_ERR_WORKSPACE
    need = P.poetx_bwd_workspace_size(d)
    assert _bwd(d, z=None, ws_bytes=need - 1) == P.POETX_ERR_WORKSPACE


def test_recompute_z_forward_workspace_holds_z():
    for act, es in ((P.POETX_BF16, 2), (P.POETX_F32, 4)):
        keep = P.poetx_fwd_workspace_size(desc(act=act, tokens=1000, d_out=4096))
        mem = P.poetx_fwd_workspace_size(desc(act=act, tokens=1000, d_out=4096,
                                              flags=P.POETX_RECOMPUTE_Z))
        assert mem - keep >= 1000 * 4096 * es
        # the backward recomputes into buffers it already has
        assert P.poetx_bwd_workspace_size(desc(act=act, tokens=1000, d_out=4096)) == \
            P.poetx_bwd_workspace_size(desc(act=act, tokens=1000, d_out=4096,
                                            flags=P.POETX_RECOMPUTE_Z))


def test_small_blocks_reserve_their_super_blocks():
    """b = 32 / 64 in bf16 with 128 | d run on 128 x 128 block-diagonal super
    blocks: both workspaces hold the larger side's super blocks (d x 128
    bf16), and the backward's gram partials are those of the super blocks;
    float32, or a d that 128 does not divide, reserve none of it."""
    def ws(b, act, d_in=4096, d_out=6144):
        d = P.make_desc(1000, d_in, d_out, b, b, act)
        return P.poetx_fwd_workspace_size(d), P.poetx_bwd_workspace_size(d)
    f128, _ = ws(128, P.POETX_BF16)
    f128_f32, _ = ws(128, P.POETX_F32)
    for b in (32, 64):
        f, bw = ws(b, P.POETX_BF16)
        assert f >= 1000 * 4096 * 2 + 6144 * 128 * 2
        assert f - 6144 * 128 * 2 <= f128
        assert bw >= 6144 * 128 * 2
        assert ws(b, P.POETX_F32)[0] == f128_f32  # float32: no super blocks
    # 128 divides neither 4032 (63 x 64) nor 4000: no super blocks
    f_odd, _ = ws(64, P.POETX_BF16, d_in=4032, d_out=4000)
    assert f_odd == 1000 * 4032 * 2


def test_recompute_z_alias_checks_skip_null_z():
    d = desc(flags=P.POETX_RECOMPUTE_Z)
    assert _fwd(d, z=None, y=ALIGNED) == P.POETX_ERR_ALIAS
    assert _bwd(d, z=None, g_x=ALIGNED) == P.POETX_ERR_ALIAS


# -- POETX_SAVED_Y (the backward takes y in place of Z) ----------------------

def test_saved_y_takes_y_in_place_of_z():
    d = desc(flags=P.POETX_SAVED_Y)
    assert _fwd(d) == P.POETX_ERR_NULL            # the forward keeps no Z
    assert _bwd(d, z=None) == P.POETX_ERR_NULL    # the backward needs y
    # validation passes up to the workspace check with z_save NULL / y given
    need = P.poetx_fwd_workspace_size(d)
    assert need > 0 and _fwd(d, z=None, ws_bytes=need - 1) == P.POETX_ERR_WORKSPACE
    need = P.poetx_bwd_workspace_size(d)
    assert need > 0 and _bwd(d, ws_bytes=need - 1) == P.POETX_ERR_WORKSPACE
    # y is an input of the backward: an output on top of it is refused
    assert _bwd(d, z=ALIGNED * 64) == P.POETX_ERR_ALIAS


def test_saved_y_refuses_what_breaks_z_equals_y_r():
    """Z = Y R needs exactly orthogonal blocks (not the truncated series),
    a kept product (not POET-Xmem) and y in block order (no permutations)."""
    perm = ALIGNED * 512
    for bad in (dict(flags=P.POETX_SAVED_Y | P.POETX_RECOMPUTE_Z),
                dict(flags=P.POETX_SAVED_Y | P.POETX_CAYLEY_NEUMANN),
                dict(flags=P.POETX_SAVED_Y, perm_in=perm, perm_out=perm + 4096)):
        d = desc(**bad)
        assert _fwd(d, z=None) == P.POETX_ERR_SHAPE
        assert _bwd(d) == P.POETX_ERR_SHAPE
        assert P.poetx_fwd_workspace_size(d) == 0 and P.poetx_bwd_workspace_size(d) == 0


def test_saved_y_forward_workspace():
    """With 256 x 256 bf16 R blocks the R-apply runs in the dense kernel and Z
    is never formed: the workspace is that of the stored-Z forward. Otherwise
    Z is formed in the workspace, as with POETX_RECOMPUTE_Z. The backward's
    workspace is the same in every mode."""
    big = dict(tokens=8192, d_in=4096, d_out=14336, b_in=256, b_out=256, act=P.POETX_BF16)
    keep = P.poetx_fwd_workspace_size(desc(**big))
    assert P.poetx_fwd_workspace_size(desc(flags=P.POETX_SAVED_Y, **big)) == keep
    assert P.poetx_bwd_workspace_size(desc(flags=P.POETX_SAVED_Y, **big)) == \
        P.poetx_bwd_workspace_size(desc(**big))
    for other in (dict(big, b_out=128), dict(big, act=P.POETX_F32), dict(big, d_out=14208)):
        keep = P.poetx_fwd_workspace_size(desc(**other))
        saved = P.poetx_fwd_workspace_size(desc(flags=P.POETX_SAVED_Y, **other))
        mem = P.poetx_fwd_workspace_size(desc(flags=P.POETX_RECOMPUTE_Z, **other))
        es = 2 if other["act"] == P.POETX_BF16 else 4
        assert saved == mem and saved - keep >= other["tokens"] * other["d_out"] * es


# -- POETX_CAYLEY_NEUMANN and poetx_build_cnp (truncated series map) ---------

def test_cnp_flag_is_valid_alone_and_with_recompute():
    for f in (P.POETX_CAYLEY_NEUMANN, P.POETX_CAYLEY_NEUMANN | P.POETX_RECOMPUTE_Z):
        d = desc(flags=f)
        assert P.poetx_fwd_workspace_size(d) > 0 and P.poetx_bwd_workspace_size(d) > 0
        # validation passes up to the workspace check
        z = None if f & P.POETX_RECOMPUTE_Z else ALIGNED * 8
        assert _bwd(d, z=z, ws_bytes=P.poetx_bwd_workspace_size(d) - 1) == P.POETX_ERR_WORKSPACE
    # the series needs no extra backward workspace
    assert P.poetx_bwd_workspace_size(desc(flags=P.POETX_CAYLEY_NEUMANN)) == \
        P.poetx_bwd_workspace_size(desc())


def test_cnp_workspace_size():
    assert P.poetx_build_cnp_workspace_size(64, 8) >= 2 * 8 * 8 * 8 * 4
    assert P.poetx_build_cnp_workspace_size(100, 12) >= 2 * 9 * 12 * 12 * 4   # padded last block
    for d, b in ((64, 6), (64, 2), (0, 8), (8, 16), (1 << 20, 8192), (64, 0)):
        assert P.poetx_build_cnp_workspace_size(d, b) == 0, (d, b)


def _cnp(theta, d, b, q, f32, act_ptr, act, ws, ws_bytes):
    return P._lib.poetx_build_cnp(theta, d, b, q, f32, act_ptr, act, ws, ws_bytes, None)


def test_build_cnp_errors():
    ok = dict(theta=ALIGNED, d=64, b=8, q=ALIGNED * 2, f32=ALIGNED * 3, act_ptr=ALIGNED * 4,
              act=P.POETX_BF16, ws=ALIGNED * 5, ws_bytes=1 << 30)

    def call(**over):
        a = dict(ok)
        a.update(over)
        return _cnp(a["theta"], a["d"], a["b"], a["q"], a["f32"], a["act_ptr"], a["act"], a["ws"],
                    a["ws_bytes"])

    assert call(act=7) == P.POETX_ERR_DTYPE
    assert call(d=0) == P.POETX_ERR_SHAPE
    assert call(b=0) == P.POETX_ERR_SHAPE
    assert call(b=128) == P.POETX_ERR_SHAPE                 # b > d
    assert call(d=1 << 20, b=8192) == P.POETX_ERR_SHAPE     # b above the maximum
    assert call(b=6) == P.POETX_ERR_ALIGN                   # b not a multiple of 4
    assert call(b=2) == P.POETX_ERR_ALIGN
    assert call(theta=None) == P.POETX_ERR_NULL
    assert call(q=None) == P.POETX_ERR_NULL
    assert call(f32=None) == P.POETX_ERR_NULL
    assert call(act_ptr=None) == P.POETX_ERR_NULL
    assert call(q=ALIGNED * 2 + 4) == P.POETX_ERR_ALIGN
    assert call(f32=ALIGNED * 3 + 8) == P.POETX_ERR_ALIGN
    assert call(ws_bytes=16) == P.POETX_ERR_WORKSPACE
    assert call(ws=None) == P.POETX_ERR_WORKSPACE
    assert call(q=ALIGNED) == P.POETX_ERR_ALIAS             # Q on top of theta
    assert call(f32=ALIGNED * 2) == P.POETX_ERR_ALIAS       # R on top of Q
    assert call(act_ptr=ALIGNED * 5) == P.POETX_ERR_ALIAS   # act copy inside the workspace
    assert call(ws=ALIGNED) == P.POETX_ERR_ALIAS            # workspace on top of theta


# -- block-mixing permutations: descriptor maps and poetx_fold_weight --------

PERMS = dict(perm_in=ALIGNED * 300, perm_out=ALIGNED * 301)


def test_permutations_both_or_neither():
    for call in (_fwd, _bwd):
        assert call(desc(perm_in=ALIGNED * 300)) == P.POETX_ERR_NULL
        assert call(desc(perm_out=ALIGNED * 301)) == P.POETX_ERR_NULL
        assert call(desc(perm_in=ALIGNED * 300 + 2, perm_out=ALIGNED * 301)) == P.POETX_ERR_ALIGN
        d = desc(**PERMS)
        need = (P.poetx_fwd_workspace_size if call is _fwd else P.poetx_bwd_workspace_size)(d)
        assert call(d, ws_bytes=need - 1) == P.POETX_ERR_WORKSPACE
    assert P.poetx_fwd_workspace_size(desc(perm_in=ALIGNED)) == 0


def test_permutation_workspace_sizes():
    es = 2
    base = desc(tokens=1000, d_in=512, d_out=768)
    perm = desc(tokens=1000, d_in=512, d_out=768, **PERMS)
    N, n, m = 1000, 512, 768
    assert P.poetx_fwd_workspace_size(perm) - P.poetx_fwd_workspace_size(base) >= N * (n + m) * es + m * 4
    assert P.poetx_bwd_workspace_size(perm) - P.poetx_bwd_workspace_size(base) >= N * (n + m) * es + n * 4


def test_permutation_maps_are_inputs_for_alias_checks():
    d = desc(**PERMS)
    assert _fwd(d, y=ALIGNED * 300) == P.POETX_ERR_ALIAS       # y on top of perm_in
    assert _bwd(d, g_x=ALIGNED * 301) == P.POETX_ERR_ALIAS     # g_x on top of perm_out


def _fold(W0, d_out, d_in, po, pi, act, out):
    return P._lib.poetx_fold_weight(W0, d_out, d_in, po, pi, act, out, None)


def test_fold_weight_errors():
    ok = dict(W0=ALIGNED, d_out=64, d_in=32, po=ALIGNED * 2, pi=ALIGNED * 3, act=P.POETX_BF16,
              out=ALIGNED * 4)

    def call(**over):
        a = dict(ok)
        a.update(over)
        return _fold(a["W0"], a["d_out"], a["d_in"], a["po"], a["pi"], a["act"], a["out"])

    assert call(act=3) == P.POETX_ERR_DTYPE
    assert call(d_out=0) == P.POETX_ERR_SHAPE
    assert call(d_in=-4) == P.POETX_ERR_SHAPE
    assert call(W0=None) == P.POETX_ERR_NULL
    assert call(po=None) == P.POETX_ERR_NULL
    assert call(pi=None) == P.POETX_ERR_NULL
    assert call(out=None) == P.POETX_ERR_NULL
    assert call(d_in=36) == P.POETX_ERR_ALIGN                # bf16 rows of 72 bytes
    assert call(out=ALIGNED * 4 + 8) == P.POETX_ERR_ALIGN
    assert call(po=ALIGNED * 2 + 2) == P.POETX_ERR_ALIGN
    assert call(out=ALIGNED) == P.POETX_ERR_ALIAS            # in place
    assert call(out=ALIGNED * 3) == P.POETX_ERR_ALIAS        # on top of perm_in


# -- INT8 frozen weight: descriptor w_scale and poetx_quantize_weight ---------

def test_int8_weight_descriptor_checks():
    for call in (_fwd, _bwd):
        assert call(desc(w_scale=ALIGNED * 310 + 2)) == P.POETX_ERR_ALIGN
        d = desc(w_scale=ALIGNED * 310, act=P.POETX_F32, d_in=60, b_in=12, b_out=4)
        assert call(d) == P.POETX_ERR_ALIGN                      # d_in not a multiple of 8
        d = desc(w_scale=ALIGNED * 310)
        need = (P.poetx_fwd_workspace_size if call is _fwd else P.poetx_bwd_workspace_size)(d)
        assert call(d, ws_bytes=need - 1) == P.POETX_ERR_WORKSPACE
    assert _fwd(desc(w_scale=ALIGNED * 64)) == P.POETX_ERR_ALIAS  # scales on top of y


def test_int8_workspace_holds_codes_and_scaled_blocks():
    # few tokens: one chunk covers the whole weight
    N, n, m, b, es = 100, 512, 768, 128, 2
    base = desc(tokens=N, d_in=n, d_out=m, b_in=b, b_out=b)
    q8 = desc(tokens=N, d_in=n, d_out=m, b_in=b, b_out=b, w_scale=ALIGNED * 310)
    # forward: the widened codes and the scaled R blocks; backward: one
    # region for both (never live together there)
    extra = m * n * es + (m // b) * b * b * es
    assert P.poetx_fwd_workspace_size(q8) - P.poetx_fwd_workspace_size(base) >= extra
    assert P.poetx_bwd_workspace_size(q8) - P.poetx_bwd_workspace_size(base) >= m * n * es


@pytest.mark.parametrize("flags", [0, P.POETX_RECOMPUTE_Z])
def test_int8_layer_holds_no_more_than_the_act_type_weight(flags):
    """The 8B MLP up-projection: the int8 codes plus the forward's workspace
    take less memory than the bf16 weight plus the same call's workspace
    without INT8, and the backward's no more, since the codes are widened a
    chunk of 4096 weight rows (forward) or 2048 columns (backward) at a time
    and the backward's chunks share their region with R's column-scaled
    blocks."""
    N, n, m, b = 8192, 4096, 14336, 256
    base = desc(tokens=N, d_in=n, d_out=m, b_in=b, b_out=b, flags=flags)
    q8 = desc(tokens=N, d_in=n, d_out=m, b_in=b, b_out=b, w_scale=ALIGNED * 310, flags=flags)
    w_bf16, w_q8 = m * n * 2, m * n
    fwd = lambda d: P.poetx_fwd_workspace_size(d)  # noqa: E731
    bwd = lambda d: P.poetx_bwd_workspace_size(d)  # noqa: E731
    assert w_q8 + fwd(q8) < w_bf16 + fwd(base)
    assert w_q8 + bwd(q8) <= w_bf16 + bwd(base)
    # exactly: forward 4096 code rows widened + the scaled R blocks; backward
    # one region of m x 2048 widened code columns (the largest of its uses,
    # also with Z recomputed: 4096 x n rows are fewer)
    align = 256
    up = lambda v: (v + align - 1) // align * align  # noqa: E731
    assert fwd(q8) - fwd(base) == up(4096 * n * 2) + up(m * b * 2)
    assert bwd(q8) - bwd(base) == up(m * 2048 * 2)


def test_quantize_weight_errors():
    ok = dict(W0=ALIGNED, d_out=64, d_in=32, act=P.POETX_BF16, q=ALIGNED * 2, sc=ALIGNED * 3)

    def call(**over):
        a = dict(ok)
        a.update(over)
        return P._lib.poetx_quantize_weight(a["W0"], a["d_out"], a["d_in"], a["act"], a["q"],
                                            a["sc"], None)

    assert call(act=5) == P.POETX_ERR_DTYPE
    assert call(d_out=0) == P.POETX_ERR_SHAPE
    assert call(d_in=0) == P.POETX_ERR_SHAPE
    assert call(W0=None) == P.POETX_ERR_NULL
    assert call(q=None) == P.POETX_ERR_NULL
    assert call(sc=None) == P.POETX_ERR_NULL
    assert call(d_in=36, act=P.POETX_F32) == P.POETX_ERR_ALIGN
    assert call(q=ALIGNED * 2 + 8) == P.POETX_ERR_ALIGN
    assert call(sc=ALIGNED * 3 + 2) == P.POETX_ERR_ALIGN
    assert call(q=ALIGNED) == P.POETX_ERR_ALIAS                 # codes on top of W0
    assert call(sc=ALIGNED * 2 + 64) == P.POETX_ERR_ALIAS       # scales inside the codes


# -- poetx_linear_fwd_noalloc: the forward with the library's fixed scratch ---

def _fwd_noalloc(desc, **over):
    args = dict(x=ALIGNED, W0=ALIGNED * 2, R=ALIGNED * 3, P=ALIGNED * 4, y=ALIGNED * 64,
                z=ALIGNED * 128)
    args.update(over)
    return P._lib.poetx_linear_fwd_noalloc(ctypes.byref(desc), args["x"], args["W0"], args["R"],
                                           args["P"], args["y"], args["z"], None)


def test_noalloc_forward_host_checks():
    """Argument faults and a workspace beyond the scratch area are reported
    before any HIP call (so they are seen here, without a GPU)."""
    assert P.POETX_NOALLOC_SCRATCH_BYTES == 64 << 20
    assert _fwd_noalloc(desc(tokens=0)) == P.POETX_ERR_SHAPE
    assert _fwd_noalloc(desc(act=5)) == P.POETX_ERR_DTYPE
    assert _fwd_noalloc(desc(), x=None) == P.POETX_ERR_NULL
    assert _fwd_noalloc(desc(), z=None) == P.POETX_ERR_NULL
    assert _fwd_noalloc(desc(flags=P.POETX_RECOMPUTE_Z)) == P.POETX_ERR_NULL  # z must be NULL then
    assert _fwd_noalloc(desc(), y=ALIGNED * 64 + 2) == P.POETX_ERR_ALIGN
    # the 8B-class MLP up-projection's forward fits exactly; one more token does not
    fits = desc(tokens=8192, d_in=4096, d_out=14336, b_in=256, b_out=256)
    assert P.poetx_fwd_workspace_size(fits) == P.POETX_NOALLOC_SCRATCH_BYTES
    over = desc(tokens=8193, d_in=4096, d_out=14336, b_in=256, b_out=256)
    assert P.poetx_fwd_workspace_size(over) > P.POETX_NOALLOC_SCRATCH_BYTES
    assert _fwd_noalloc(over) == P.POETX_ERR_WORKSPACE
    # POET-Xmem keeps Z in the forward's workspace: too large here
    mem = desc(tokens=8192, d_in=4096, d_out=14336, b_in=256, b_out=256, flags=P.POETX_RECOMPUTE_Z)
    assert _fwd_noalloc(mem, z=None) == P.POETX_ERR_WORKSPACE
