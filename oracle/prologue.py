"""Oracle of the Q/K prologue in front of the block-sparse path: RMSNorm, then 3-D rotary
position embedding (test infrastructure: imported only by the tests, the smoke run and the
benchmark's CPU baseline).

Page "600倍加速，720p视频实时生成！单卡也能带的动14B模型", efficient inference operators
paragraph, and page "Run Wan2.2-A14B on One RTX 5090: 720p Video in 3.8s", section 4: 3-D RoPE
and RMSNorm run as fused or parallel kernels. The pages do not define either operation; the
readings, from their published definitions:

* RMSNorm (Zhang and Sennrich, 2019): y_c = x_c / sqrt(mean_c x_c^2 + eps) * g_c over the d
  channels of one head's row (a per-head norm of Q and of K, with a gain g per head and
  channel).
* 3-D RoPE: the rotary embedding of Su et al. (RoFormer, 2021) rotates adjacent channel pairs
  (x_2p, x_2p+1) by an angle proportional to the position; for a video latent the d/2 pairs are
  split over the three grid axes, as evenly as possible with the extra pairs on the time axis
  (d = 128: 22 pairs for the frame t, 21 for the row y, 21 for the column x). Pair j of an
  axis group of n pairs turns by pos * theta^(-j/n), theta = 10000, with (t, y, x) the grid
  coordinates of the token (row-major flattening, as for the blocks). (x0, x1) becomes
  (x0 cos a - x1 sin a, x0 sin a + x1 cos a).
* Precision: the prologue's output decides the INT8/FP8 codes, so it is computed in the
  precision the kernel takes that decision in: fp32, each IEEE operation rounded on its own.
  The mean square is the exact fp64 sum of the squares (exact for bf16 inputs), divided by d
  and rounded to fp32; then r = 1 / sqrt(ms + eps) (eps rounded to fp32), y = (x * r) * g;
  cos and sin of every angle are taken in fp64 and rounded to fp32; the rotation's products
  and their sum are fp32 operations. Written this way the result is a function of the IEEE
  operations alone, so a kernel doing the same operations reproduces it bit for bit.
  rms_norm64 / rope3d64 are the same definitions in fp64; the pins tie the fp32 result to them
  within fp32's error bound.

Parity unpinned against the pages (they define neither operation); pinned to the published
definitions by tests/test_oracle_pins.py (torch's rms_norm, complex multiplication, closed
forms, a hand example).
"""
import numpy as np


def rms_norm64(X, g, eps: float):
    """X [B, H, L, d], g [H, d]: RMSNorm over the last axis, in fp64."""
    X = np.asarray(X, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    return X / np.sqrt(np.mean(X * X, axis=-1, keepdims=True) + eps) * g[None, :, None, :]


def rms_norm(X, g, eps: float):
    """X [B, H, L, d] (fp32 values), g [H, d]: RMSNorm over the last axis in fp32 operations, the
    mean square from the exact fp64 sum of the squares."""
    X = np.asarray(X, dtype=np.float32)
    g = np.asarray(g, dtype=np.float32)
    x64 = X.astype(np.float64)
    ms = (np.sum(x64 * x64, axis=-1, keepdims=True) / X.shape[-1]).astype(np.float32)
    r = np.float32(1.0) / np.sqrt(ms + np.float32(eps))
    return (X * r) * g[None, :, None, :]


def axis_pairs(d: int):
    """Pairs per grid axis (t, y, x): d/2 split as evenly as possible, the rest to t."""
    n = d // 2
    base = n // 3
    return (n - 2 * base, base, base)


def grid_positions(grid, L: int):
    """(t, y, x) of every token n < L on a (T, Hg, Wg) grid, row-major."""
    T, Hg, Wg = grid
    n = np.arange(L)
    return n // (Hg * Wg), (n // Wg) % Hg, n % Wg


def rope_cos_sin(grid, L: int, d: int, theta: float = 10000.0):
    """cos and sin, rounded to fp32, of the angle of every (token, pair): two [L, d/2] arrays."""
    pos = grid_positions(grid, L)
    ang = np.empty((L, d // 2), np.float64)
    p0 = 0
    for axis, n in enumerate(axis_pairs(d)):
        j = np.arange(n, dtype=np.float64)
        freq = theta ** (-j / n)
        ang[:, p0:p0 + n] = pos[axis][:, None].astype(np.float64) * freq[None, :]
        p0 += n
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rope3d(X, grid, theta: float = 10000.0):
    """X [B, H, L, d]: rotate adjacent channel pairs by the token's 3-D angles, in fp32."""
    X = np.asarray(X, dtype=np.float32)
    L, d = X.shape[2], X.shape[3]
    c, s = rope_cos_sin(grid, L, d, theta)
    c, s = c[None, None], s[None, None]
    x0, x1 = X[..., 0::2], X[..., 1::2]
    out = np.empty_like(X)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def rope3d64(X, grid, theta: float = 10000.0):
    """The same rotation in fp64, with the angles' cos and sin in fp64."""
    X = np.asarray(X, dtype=np.float64)
    L, d = X.shape[2], X.shape[3]
    pos = grid_positions(grid, L)
    ang = np.concatenate([pos[a][:, None].astype(np.float64) * theta ** (-np.arange(n) / n)[None, :]
                          for a, n in enumerate(axis_pairs(d))], axis=1)
    c, s = np.cos(ang)[None, None], np.sin(ang)[None, None]
    out = np.empty_like(X)
    out[..., 0::2] = X[..., 0::2] * c - X[..., 1::2] * s
    out[..., 1::2] = X[..., 0::2] * s + X[..., 1::2] * c
    return out


def qk_prologue(X, g, eps: float, grid, theta: float = 10000.0):
    """RMSNorm then 3-D RoPE of Q or K ([B, H, L, d], bf16 values), fp32 result."""
    return rope3d(rms_norm(X, g, eps), grid, theta)


def qk_prologue64(X, g, eps: float, grid, theta: float = 10000.0):
    """The fp64 definitions (RMSNorm then 3-D RoPE) and, per element, a bound on how far the fp32
    operation sequence of qk_prologue can land from them: 8 * 2^-24 of the pair's |y0| + |y1|
    (the norm's square root, reciprocal and two products, then a rotation's two products and
    its sum, each one fp32 rounding, with a factor of two to spare).
    Returns (Y64, bound), float64 [B, H, L, d]."""
    Y = rope3d64(rms_norm64(X, g, eps), grid, theta)
    pair = np.abs(Y[..., 0::2]) + np.abs(Y[..., 1::2])
    return Y, 8 * 2.0 ** -24 * np.repeat(pair, 2, axis=-1)
