"""Seeded synthetic inputs for the POET-X linear layer.

This module is shared by the oracle-side tests, the GPU parity tests and the
benchmark. It holds no arithmetic of the method itself: it only draws random
numbers, scales them and rounds them to the storage precision of a workload.

Workloads. The pages train Llama-style models of 3B, 8B and 13B parameters on
C4 (gist.science summary of POET-X, "Technische Zusammenfassung" §4
Ergebnisse). Neither the data nor trained weights are needed to exercise the
layer: the synthetic layers below stand in for them with the shapes of those
models' projections (hidden 2048 for a 1B-class model; hidden 4096, MLP 14336
and grouped-query k/v width 1024 for the 8B class; block size 512 as in the
perplexity experiment of §4).

Recipe (one layer):
  rng = numpy.random.default_rng(seed)  (PCG64)
  draw standard normals in float64 in the order W0 [d_out, d_in],
  theta_R [nb_R, b(b-1)/2], theta_P [nb_P, b(b-1)/2], x [tokens, d_in],
  g_y [tokens, d_out];
  scale W0 by 1/sqrt(d_in) and theta by sigma_theta;
  round theta to float32 (round-to-nearest-even), and W0, x, g_y to the
  activation dtype: float32 (RNE) or bfloat16 (float64 -> float32 RNE ->
  bfloat16 RNE).
The arrays returned are float64 arrays holding exactly the rounded values, so
the oracle consumes the very numbers the GPU path is given. Where R and P have
different block sizes (make_layer_blocks), theta_R has b_out(b_out-1)/2 entries
per block and theta_P b_in(b_in-1)/2; the order and scaling are the same.

Block-mixing permutations (when a test or the benchmark uses them) are drawn
from their own generator, numpy.random.default_rng(seed + 7919):
perm_out = permutation(d_out), then perm_in = permutation(d_in), int32.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List

import numpy as np

__all__ = [
    "LayerSpec", "LayerInputs", "CONFIGS", "config_layers", "make_layer",
    "round_to_dtype", "bf16_bits", "num_blocks", "theta_count", "resized",
    "make_permutations", "make_layer_blocks",
]


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """Shape and distribution of one synthetic POET-X linear layer."""
    name: str
    d_in: int
    d_out: int
    b: int                 # block size of both R (on d_out) and P (on d_in)
    tokens: int
    dtype: str             # "f32" or "bf16": storage type of W0, x, y, g_y, g_x
    sigma_theta: float
    seed: int

    @property
    def nb_out(self) -> int:
        return num_blocks(self.d_out, self.b)

    @property
    def nb_in(self) -> int:
        return num_blocks(self.d_in, self.b)

    @property
    def tri(self) -> int:
        return self.b * (self.b - 1) // 2


@dataclasses.dataclass
class LayerInputs:
    spec: LayerSpec
    W0: np.ndarray        # [d_out, d_in] float64 (values exact in spec.dtype)
    theta_R: np.ndarray   # [nb_out, b(b-1)/2] float64 (values exact in float32)
    theta_P: np.ndarray   # [nb_in,  b(b-1)/2] float64 (values exact in float32)
    x: np.ndarray         # [tokens, d_in]
    g_y: np.ndarray       # [tokens, d_out]


def num_blocks(d: int, b: int) -> int:
    return -(-d // b)


def theta_count(d: int, b: int) -> int:
    return num_blocks(d, b) * (b * (b - 1) // 2)


def _round_f32(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float64 data: float32 RNE, then bfloat16 RNE."""
    f = _round_f32(a)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    rounded = rounded.astype(np.uint16)
    rounded[nan] = 0x7FC0
    return rounded


def round_to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 data to `dtype` storage and return the values as float64."""
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    if dtype == "f32":
        return _round_f32(a).astype(np.float64)
    if dtype == "bf16":
        bits = bf16_bits(a).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_layer(spec: LayerSpec) -> LayerInputs:
    """Draw one layer's inputs by the recipe in the module docstring."""
    rng = np.random.default_rng(spec.seed)
    n, m = spec.d_in, spec.d_out
    W0 = rng.standard_normal((m, n)) / math.sqrt(n)
    thR = rng.standard_normal((spec.nb_out, spec.tri)) * spec.sigma_theta
    thP = rng.standard_normal((spec.nb_in, spec.tri)) * spec.sigma_theta
    x = rng.standard_normal((spec.tokens, n))
    g_y = rng.standard_normal((spec.tokens, m))
    act = spec.dtype
    return LayerInputs(
        spec=spec,
        W0=round_to_dtype(W0, act),
        theta_R=round_to_dtype(thR, "f32"),
        theta_P=round_to_dtype(thP, "f32"),
        x=round_to_dtype(x, act),
        g_y=round_to_dtype(g_y, act),
    )


def make_layer_blocks(d_in: int, d_out: int, b_in: int, b_out: int, tokens: int, dtype: str,
                      sigma_theta: float, seed: int) -> Dict[str, np.ndarray]:
    """One layer whose R (on d_out) and P (on d_in) have their own block sizes,
    drawn by the same recipe: a dict with W0, theta_R, theta_P, x and g_y."""
    rng = np.random.default_rng(seed)
    tri_out, tri_in = b_out * (b_out - 1) // 2, b_in * (b_in - 1) // 2
    W0 = rng.standard_normal((d_out, d_in)) / math.sqrt(d_in)
    thR = rng.standard_normal((num_blocks(d_out, b_out), tri_out)) * sigma_theta
    thP = rng.standard_normal((num_blocks(d_in, b_in), tri_in)) * sigma_theta
    x = rng.standard_normal((tokens, d_in))
    g_y = rng.standard_normal((tokens, d_out))
    return {"W0": round_to_dtype(W0, dtype), "theta_R": round_to_dtype(thR, "f32"),
            "theta_P": round_to_dtype(thP, "f32"), "x": round_to_dtype(x, dtype),
            "g_y": round_to_dtype(g_y, dtype)}


def make_permutations(spec: LayerSpec):
    """Seeded random index maps (perm_out [d_out], perm_in [d_in]), int32."""
    rng = np.random.default_rng(spec.seed + 7919)
    perm_out = rng.permutation(spec.d_out).astype(np.int32)
    perm_in = rng.permutation(spec.d_in).astype(np.int32)
    return perm_out, perm_in


def resized(spec: LayerSpec, **changes) -> LayerSpec:
    """A copy of `spec` with some fields changed (a different, usually smaller,
    layer drawn by the same recipe)."""
    return dataclasses.replace(spec, **changes)


def _layer(name, d_in, d_out, b, tokens, dtype, sigma, seed) -> LayerSpec:
    return LayerSpec(name, d_in, d_out, b, tokens, dtype, sigma, seed)


# The five workloads. Each entry is the list of layers that one step runs.
CONFIGS: Dict[str, List[LayerSpec]] = {
    # Tiny fp32 layer: d 256, b 32 (8 blocks each side), 64 tokens.
    "tiny_f32": [_layer("tiny", 256, 256, 32, 64, "f32", 0.02, 0)],
    # 1B-class projection: 2048 x 2048, b 256, 8192 tokens (4 x 2048).
    "proj_1b": [_layer("proj", 2048, 2048, 256, 8192, "bf16", 0.01, 0)],
    # 8B-class MLP up-projection: W0 14336 x 4096 (out x in), b 256, 8192 tokens.
    "mlp_up_8b": [_layer("up", 4096, 14336, 256, 8192, "bf16", 0.01, 0)],
    # 8B-class set of seven projections, b 512, 16384 tokens (8 x 2048).
    "layer_set_8b": [
        _layer("q", 4096, 4096, 512, 16384, "bf16", 0.01, 0),
        _layer("k", 4096, 1024, 512, 16384, "bf16", 0.01, 1),
        _layer("v", 4096, 1024, 512, 16384, "bf16", 0.01, 2),
        _layer("o", 4096, 4096, 512, 16384, "bf16", 0.01, 3),
        _layer("gate", 4096, 14336, 512, 16384, "bf16", 0.01, 4),
        _layer("up", 4096, 14336, 512, 16384, "bf16", 0.01, 5),
        _layer("down", 14336, 4096, 512, 16384, "bf16", 0.01, 6),
    ],
}
for _b in (64, 128, 256, 512, 1024):
    CONFIGS[f"sweep_b{_b}"] = [_layer(f"sq_b{_b}", 4096, 4096, _b, 8192, "bf16", 0.01, 0)]


def config_layers(name: str) -> List[LayerSpec]:
    return list(CONFIGS[name])
