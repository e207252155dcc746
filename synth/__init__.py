"""Seeded synthetic Q/K/V on a 3-D video-latent token grid.

This module only draws random numbers and lays them out. It holds none of the
attention method's arithmetic, so both the CPU oracle's tests and the GPU path
can take their inputs from it without sharing any computation.

The recipe (the pages fix none of it; the shapes are those of the 480p/720p
Wan2.2 latents the pages talk about, page "600倍加速，720p视频实时生成！",
section on why generation is slow, which puts the sequence near 120K tokens):

* tokens sit on a (T, Hg, Wg) grid and are flattened row-major,
  n = (t*Hg + y)*Wg + x;
* per (batch, head) a generator seeded with (seed, b, h) draws, in order,
  8 integer wave vectors in {0,1,2}^3 (an all-zero one becomes (0,0,1)),
  8 phases in [0, 2*pi), an 8 x d amplitude matrix A ~ N(0,1), then the
  Q noise, the K noise and V, each L x d;
* feat[n, f] = cos(2*pi*(k_f . (t/T, y/Hg, x/Wg)) + phi_f);
* Q = feat @ A + sigma*N(0,1),  K = feat @ A + sigma*N(0,1),  V = N(0,1).

Q and K share the wave vectors, phases and amplitudes, so nearby key blocks
score high for a query block, the structure that makes block selection pay.
"""
from .grid import CONFIGS, GridConfig, grid_features, head_qkv, make_qkv, wide_rows  # noqa: F401
