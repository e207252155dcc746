"""Seeded generator for the synthetic grid workloads (no attention arithmetic here)."""
from __future__ import annotations

import dataclasses
import math

import numpy as np

N_FEATURES = 8


@dataclasses.dataclass(frozen=True)
class GridConfig:
    """One workload: shape, token grid, block sizes, keep ratio(s) and noise."""

    name: str
    B: int
    H: int
    grid: tuple  # (T, Hg, Wg)
    d: int
    block_q: int
    block_k: int
    keeps: tuple  # keep ratios the workload is run at
    sigmas: tuple  # noise std per batch item
    in_dtype: str  # "fp32" or "bf16"
    mode: str  # "bf16" or "int8fp8"
    seed: int

    @property
    def L(self) -> int:
        T, Hg, Wg = self.grid
        return T * Hg * Wg

    @property
    def keep(self) -> float:
        return self.keeps[0]


# Shapes of the workloads the method is measured on: a tiny case the oracle
# runs in full, a 480p-shaped bf16 case, the 720p-shaped quantized case (the
# headline), the ~120K-token case and a keep-ratio sweep over two noise levels.
CONFIGS = {
    "tiny": GridConfig("tiny", 1, 2, (4, 16, 16), 128, 64, 64, (0.25,), (0.5,),
                       "fp32", "bf16", 0),
    "480p": GridConfig("480p", 1, 40, (21, 30, 52), 128, 128, 64, (0.2,), (0.5,),
                       "bf16", "bf16", 1),
    "720p": GridConfig("720p", 1, 40, (21, 45, 80), 128, 128, 64, (0.1,), (0.5,),
                       "bf16", "int8fp8", 2),
    "long": GridConfig("long", 1, 40, (30, 64, 64), 128, 128, 64, (0.1, 1.0), (0.5,),
                       "bf16", "int8fp8", 3),
    "sweep": GridConfig("sweep", 2, 40, (21, 45, 80), 128, 128, 64,
                        (0.05, 0.1, 0.2, 0.5, 1.0), (0.25, 1.0), "bf16", "int8fp8", 4),
}


def grid_features(grid, kvec, phi):
    """feat[n, f] = cos(2*pi*(k_f . (t/T, y/Hg, x/Wg)) + phi_f), float64 [L, F]."""
    T, Hg, Wg = grid
    t = np.arange(T, dtype=np.float64) / T
    y = np.arange(Hg, dtype=np.float64) / Hg
    x = np.arange(Wg, dtype=np.float64) / Wg
    tt, yy, xx = np.meshgrid(t, y, x, indexing="ij")
    coords = np.stack([tt.ravel(), yy.ravel(), xx.ravel()], axis=1)  # [L, 3], row-major
    return np.cos(2.0 * math.pi * (coords @ kvec.T.astype(np.float64)) + phi[None, :])


def head_qkv(seed: int, b: int, h: int, grid, d: int, sigma: float):
    """Q, K, V for one (batch, head) as float32 [L, d] arrays.

    Each head has its own generator seeded with (seed, b, h), so any head can be
    drawn alone (the oracle's sampled heads) and the draw does not depend on B or H.
    """
    rng = np.random.default_rng([seed, b, h])
    kvec = rng.integers(0, 3, size=(N_FEATURES, 3))
    kvec[np.all(kvec == 0, axis=1)] = (0, 0, 1)
    phi = rng.uniform(0.0, 2.0 * math.pi, size=N_FEATURES)
    A = rng.standard_normal((N_FEATURES, d))
    L = int(np.prod(grid))
    base = (grid_features(grid, kvec, phi) @ A).astype(np.float32)
    q = base + np.float32(sigma) * rng.standard_normal((L, d), dtype=np.float32)
    k = base + np.float32(sigma) * rng.standard_normal((L, d), dtype=np.float32)
    v = rng.standard_normal((L, d), dtype=np.float32)
    return q, k, v


def make_qkv(cfg: GridConfig, heads=None, batches=None):
    """Q, K, V as float32 numpy arrays [B', H', L, d] for the chosen (b, h) subset.

    Inputs of bf16 workloads are rounded to bf16 by the caller (torch's RNE cast);
    this module returns the float32 draw.
    """
    heads = list(range(cfg.H)) if heads is None else list(heads)
    batches = list(range(cfg.B)) if batches is None else list(batches)
    L, d = cfg.L, cfg.d
    out = [np.empty((len(batches), len(heads), L, d), np.float32) for _ in range(3)]
    for bi, b in enumerate(batches):
        sigma = cfg.sigmas[b % len(cfg.sigmas)]
        for hi, h in enumerate(heads):
            q, k, v = head_qkv(cfg.seed, b, h, cfg.grid, d, sigma)
            out[0][bi, hi], out[1][bi, hi], out[2][bi, hi] = q, k, v
    return tuple(out)


def wide_rows(seed: int, shape, zero_rows: int = 3):
    """float32 array of `shape` whose last-axis rows have magnitudes spread over ~2^-40 .. 2^40:
    N(0,1) values times a per-row factor exp2(U(-40, 40)), with `zero_rows` rows set to zero
    and one row holding a single nonzero value. Exercises per-row scaling at the edges."""
    r = np.random.default_rng(seed)
    x = r.standard_normal(shape).astype(np.float32)
    rows = x.reshape(-1, shape[-1])
    rows *= np.exp2(r.uniform(-40.0, 40.0, (rows.shape[0], 1))).astype(np.float32)
    pick = r.choice(rows.shape[0], size=min(zero_rows + 1, rows.shape[0]), replace=False)
    rows[pick[:-1]] = 0.0
    rows[pick[-1]] = 0.0
    rows[pick[-1], r.integers(shape[-1])] = -3.0
    return x
