"""Helpers for the GPU parity tests: device tensors from seeded inputs,
running one layer through libpoetx, and error metrics."""
from __future__ import annotations

import sys

import numpy as np
import torch

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """float64 values that are exact in `dtype` -> device tensor of that dtype."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(TORCH_DT[dtype]).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def max_rel(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| (the float32-path metric)."""
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))


def fro_rel(got: np.ndarray, ref: np.ndarray) -> float:
    """||got - ref||_F / ||ref||_F (the bf16-path metric)."""
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


# Tolerances: float32 path 1e-4 max-relative; bf16 storage with float32
# accumulation 2e-2 Frobenius-relative.
TOL = {"f32": (max_rel, 1e-4), "bf16": (fro_rel, 2e-2)}


def check(name: str, got, ref, dtype: str) -> float:
    metric, tol = TOL[dtype]
    err = metric(np.asarray(got), np.asarray(ref))
    log(f"    {name:10s} {metric.__name__} = {err:.3e} (tol {tol:.0e})")
    assert np.all(np.isfinite(got)), name
    assert err <= tol, (name, err, tol)
    return err


def check_tiles(name: str, got, ref, dtype: str, tile=(256, 256)) -> float:
    """Element-by-element comparison of a whole 2-D output: the tolerance
    metric over the whole tensor and over every tile x tile piece (so one
    wrong output tile cannot hide in the norm of a large tensor), plus the
    max-abs error relative to max |ref| for the log."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), name
    metric, tol = TOL[dtype]
    whole = metric(got, ref)
    worst, where = 0.0, None
    r0, c0 = tile
    for i in range(0, ref.shape[0], r0):
        for j in range(0, ref.shape[1], c0):
            e = metric(got[i:i + r0, j:j + c0], ref[i:i + r0, j:j + c0])
            if e > worst:
                worst, where = e, (i, j)
    mx = max_rel(got, ref)
    log(f"    {name:10s} {metric.__name__} = {whole:.3e}, worst {r0}x{c0} tile {worst:.3e} at {where}, "
        f"max-abs/max|ref| = {mx:.3e} (tol {tol:.0e})")
    assert whole <= tol, (name, whole, tol)
    assert worst <= tol, (name, "tile", where, worst, tol)
    return whole


def check_blocks(name: str, got, ref, dtype: str) -> float:
    """Per-block comparison of a [nblocks, ...] output (every generator
    block of g_theta), with the metric over the whole tensor as well."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), name
    metric, tol = TOL[dtype]
    whole = metric(got, ref)
    errs = [metric(got[k], ref[k]) for k in range(ref.shape[0])]
    k = int(np.argmax(errs))
    log(f"    {name:10s} {metric.__name__} = {whole:.3e}, worst of {len(errs)} blocks {errs[k]:.3e} "
        f"(block {k}), max-abs/max|ref| = {max_rel(got, ref):.3e} (tol {tol:.0e})")
    assert whole <= tol, (name, whole, tol)
    assert errs[k] <= tol, (name, "block", k, errs[k], tol)
    return whole


def run_layer(L, stream=None, recompute_z=False, map="cayley", perms=None, saved_y=False,
              int8=False):
    """Build, forward and backward one layer on the GPU (the bench's path).
    Returns the PoetxLinear and a dict of device results (z is None when the
    layer keeps no Z: recomputed in the backward, or y kept in its place).
    perms: (perm_out, perm_in) or None."""
    from orthogonal_equivalence_amd.layer import PoetxLinear
    s = L.spec
    po, pi = perms if perms is not None else (None, None)
    lay = PoetxLinear(dev(L.W0, s.dtype), s.b, s.b, s.dtype, recompute_z=recompute_z, map=map,
                      perm_out=po, perm_in=pi, saved_y=saved_y, int8=int8)
    lay.set_theta(torch.from_numpy(L.theta_R).float(), torch.from_numpy(L.theta_P).float())
    x = dev(L.x, s.dtype)
    g_y = dev(L.g_y, s.dtype)
    lay.build(stream)
    y, z = lay.forward(x, stream=stream)
    g_x, gR, gP = lay.backward(g_y, x, z, stream=stream)
    torch.cuda.synchronize()
    return lay, dict(x=x, g_y=g_y, y=y, z=None if saved_y else z, g_x=g_x, g_theta_R=gR,
                     g_theta_P=gP)
