"""Seeded synthetic workloads for the tile-hybrid dense / 2:4 matmul.

This module only draws inputs: weight and activation bit patterns, per-tile
dense/sparse maps and per-matrix sparse-tile fractions.  It holds none of the
method's arithmetic (no pruning, packing or products), so both the HIP path and
the CPU oracle can be fed from it without sharing any code with each other.

The shapes stand in for the projection matrices the pages name:
  * PATCH (gist.science, "PATCH: Learnable Tile-level Hybrid Sparsity for
    LLMs"), section 2 "Meccanismo Principale": a weight matrix cut into b1 x b2
    tiles, each dense or 2:4 sparse; section 4: tile execution size 128 x 128.
  * SparseDecoding (ai.info, authors' abstract): decode-time sparse
    matrix x vector products on Llama-3.1-8B, Llama-3.3-70B and Qwen3-14B/32B.
No checkpoint or dataset is read; values are iid normal, so the six 2:4
patterns are equally likely and the tile map is the only structure.

Seeding: numpy.random.default_rng([config, matrix_index, role]) with role
0 = weights, 1 = activations, 2 = tile map, 3 = per-matrix fractions.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ROLE_W, ROLE_X, ROLE_MAP, ROLE_FRAC = 0, 1, 2, 3

DTYPE_CODES = {"f16": 1, "bf16": 2}


def _rng(config: int, index: int, role: int) -> np.random.Generator:
    return np.random.default_rng([int(config), int(index), int(role)])


def float32_to_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the 16-bit type with round-to-nearest-even and
    return the raw 16-bit patterns (uint16).  Inputs here are finite."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f16":
        return a.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = a.view(np.uint32).astype(np.uint64)
        rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return rounded.astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def normal_bits(config: int, index: int, role: int, shape, sigma: float, dtype: str) -> np.ndarray:
    """iid N(0, sigma) drawn in float32 and rounded to `dtype` bit patterns."""
    g = _rng(config, index, role)
    vals = g.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        vals *= np.float32(sigma)
    return float32_to_bits(vals, dtype)


def n_sparse_for_fraction(n_tiles: int, frac: float) -> int:
    """Sparse tile count for a target fraction: nearest integer, halves up."""
    return int(np.floor(frac * n_tiles + 0.5))


def tile_map_random(config: int, index: int, tiles_n: int, tiles_k: int, frac: float) -> np.ndarray:
    """uint8[tiles_n, tiles_k]; the first n_sparse tiles of a seeded
    permutation of the row-major tile ids are sparse (1), the rest dense (0)."""
    total = tiles_n * tiles_k
    ns = n_sparse_for_fraction(total, frac)
    perm = _rng(config, index, ROLE_MAP).permutation(total)
    m = np.zeros(total, dtype=np.uint8)
    m[perm[:ns]] = 1
    return m.reshape(tiles_n, tiles_k)


def tile_map_checkerboard(config: int, index: int, tiles_n: int, tiles_k: int) -> np.ndarray:
    """Seeded checkerboard: tile (tn, tk) is sparse iff (tn + tk + p) is even,
    with the parity bit p drawn from the seed."""
    p = int(_rng(config, index, ROLE_MAP).integers(2))
    tn = np.arange(tiles_n)[:, None]
    tk = np.arange(tiles_k)[None, :]
    return (((tn + tk + p) % 2) == 0).astype(np.uint8)


def tile_map_const(tiles_n: int, tiles_k: int, value: int) -> np.ndarray:
    return np.full((tiles_n, tiles_k), value, dtype=np.uint8)


@dataclass
class Matrix:
    """One weight matrix of a workload: W is n x k (out x in), tile b1 x b2."""
    name: str
    n: int
    k: int
    b1: int
    b2: int
    dtype: str
    sigma: float
    config: int
    index: int
    frac: float | None = None          # sparse-tile fraction (random placement)
    placement: str = "random"          # "random" | "checkerboard" | "const"

    @property
    def tiles_n(self) -> int:
        return self.n // self.b1

    @property
    def tiles_k(self) -> int:
        return self.k // self.b2

    def weight_bits(self) -> np.ndarray:
        return normal_bits(self.config, self.index, ROLE_W, (self.n, self.k), self.sigma, self.dtype)

    def activation_bits(self, m: int) -> np.ndarray:
        return normal_bits(self.config, self.index, ROLE_X, (m, self.k), 1.0, self.dtype)

    def tile_map(self) -> np.ndarray:
        if self.placement == "checkerboard":
            return tile_map_checkerboard(self.config, self.index, self.tiles_n, self.tiles_k)
        if self.placement == "const":
            return tile_map_const(self.tiles_n, self.tiles_k, 1 if self.frac else 0)
        return tile_map_random(self.config, self.index, self.tiles_n, self.tiles_k, self.frac)


@dataclass
class Workload:
    config: int
    title: str
    matrices: list = field(default_factory=list)
    batches: tuple = (1,)


def layer_fractions(config: int = 3) -> np.ndarray:
    """Seven iid U(0.2, 0.8) sparse-tile fractions, in the order
    q, k, v, o, gate, up, down (the mean 0.5 is the law's, not enforced)."""
    return _rng(config, 0, ROLE_FRAC).uniform(0.2, 0.8, size=7)


def workload(config: int) -> Workload:
    """The five synthetic workloads, numbered as in the benchmark plan."""
    if config == 1:
        return Workload(1, "512x512 fp16, 8 of 16 tiles 2:4 (25% sparsity)",
                        [Matrix("w", 512, 512, 128, 128, "f16", 0.02, 1, 0, frac=0.5)], (1,))
    if config == 2:
        return Workload(2, "Llama-3.1-8B up projection 14336x4096 bf16, 70% sparse tiles",
                        [Matrix("up", 14336, 4096, 128, 128, "bf16", 0.02, 2, 0, frac=0.7)], (1,))
    if config == 3:
        fr = layer_fractions(3)
        shapes = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
                  ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336)]
        mats = [Matrix(nm, n, k, 128, 128, "bf16", 0.02, 3, j, frac=float(fr[j]))
                for j, (nm, n, k) in enumerate(shapes)]
        return Workload(3, "Llama-3.1-8B decoder layer, per-matrix fractions U(0.2,0.8)", mats, (1, 4, 16))
    if config == 4:
        mats = []
        for j, (nm, n, k) in enumerate([("wide", 28672, 8192), ("tall", 8192, 28672)]):
            mats.append(Matrix(f"{nm}_dense", n, k, 128, 128, "bf16", 0.015, 4, j, frac=0.0, placement="const"))
            mats.append(Matrix(f"{nm}_sparse", n, k, 128, 128, "bf16", 0.015, 4, j, frac=1.0, placement="const"))
            mats.append(Matrix(f"{nm}_checker", n, k, 128, 128, "bf16", 0.015, 4, j, placement="checkerboard"))
        return Workload(4, "Llama-3.3-70B MLP endpoints, 0% / 100% / checkerboard sparse tiles", mats, (1,))
    if config == 5:
        return Workload(5, "Qwen3-14B gate/up 17408x5120 bf16, 64x64 tiles, 60% sparse tiles",
                        [Matrix("gateup", 17408, 5120, 64, 64, "bf16", 0.02, 5, 0, frac=0.6)],
                        (16, 64, 256, 2048))
    raise ValueError(f"no workload {config}")
