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


def run_layer(L, stream=None, recompute_z=False, map="cayley", perms=None):
    """Build, forward and backward one layer on the GPU (the bench's path).
    Returns the PoetxLinear and a dict of device results (z is None when the
    layer recomputes Z in the backward). perms: (perm_out, perm_in) or None."""
    from orthogonal_equivalence_amd.layer import PoetxLinear
    s = L.spec
    po, pi = perms if perms is not None else (None, None)
    lay = PoetxLinear(dev(L.W0, s.dtype), s.b, s.b, s.dtype, recompute_z=recompute_z, map=map,
                      perm_out=po, perm_in=pi)
    lay.set_theta(torch.from_numpy(L.theta_R).float(), torch.from_numpy(L.theta_P).float())
    x = dev(L.x, s.dtype)
    g_y = dev(L.g_y, s.dtype)
    lay.build(stream)
    y, z = lay.forward(x, stream=stream)
    g_x, gR, gP = lay.backward(g_y, x, z, stream=stream)
    torch.cuda.synchronize()
    return lay, dict(x=x, g_y=g_y, y=y, z=z, g_x=g_x, g_theta_R=gR, g_theta_P=gP)
