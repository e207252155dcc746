"""Oracle of the block-scaled 4-bit GEMM (NVFP4 x NVFP4, fp32 accumulation, bf16 output, column
bias) - test infrastructure: imported only by the tests, the smoke run and the benchmark's CPU
baseline.

Page "600倍加速，720p视频实时生成！单卡也能带的动14B模型", single-card path, paragraph on
NVFP4 quantization-aware training (the format: E2M1 4-bit values, one FP8 E4M3 scale per 16
consecutive elements, one FP32 scale for the whole tensor) and paragraph on efficient inference
operators (linear, MLP and MoE layers as block-scaled GEMMs with weights and activations both
in NVFP4, FP32 accumulation, BF16 output, the column bias fused into the epilogue).

Readings (the pages fix the format but not the encoding rule):

* Blocks run along the contraction axis K (16 consecutive elements of a row).
* Tensor scale S = amax / (6 * 448) (fp32 division; S = 1 for an all-zero tensor), so that the
  largest block scale is about the largest E4M3 value.
* Block scale s_b = E4M3_RNE(min(amax_b / (6 * S), 448)) with 6 * S rounded to fp32 first (a
  block's largest element maps to about 6, the largest E2M1 value; the fp32 rounding of S can
  put the largest block a hair above 448); 0 for an all-zero block.
* Element code q = E2M1_RNE(x * inv_b) with inv_b = 1 / fp32(s_b * S) (one IEEE fp32 division
  per block, then an fp32 product per element), saturating at +-6; q = 0 where s_b = 0. This is
  the convention of the INT8 quantizer reading of the attention path (one reciprocal scale per
  block, one product per element); a per-element division differs on elements at exact E2M1
  midpoints of their block (pinned in the tests). E2M1 values: 0, 0.5, 1, 1.5, 2, 3, 4, 6 and
  their negatives; ties go to the even mantissa bit; the sign of a zero result is kept.
* The element stands for q * s_b * S. The GEMM is Y[m, n] = S_A * S_W * sum_k (q_A s_A)(q_W s_W)
  + bias[n] (bias read as given, e.g. from bf16), taken here in fp64 (each product, of values with
  at most 6 significant bits each, is exact; the fp64 sum's rounding is far below the fp32
  accumulation bound the kernel is held to) and rounded to bf16 at the end.

All fp32 steps are the IEEE operations written above, so a kernel doing the same operations
produces the same codes and scales bit for bit. Parity unpinned against the pages (they print
no example); pinned to the definitions by tests/test_oracle_pins.py.
"""
import numpy as np

from .blocksparse import e4m3_rne

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float64)
BLOCK = 16


def e2m1_rne(v):
    """Round fp32 values to the E2M1 grid, ties to the even mantissa bit, saturating at +-6.
    Returns grid values (float32, sign kept, -0.0 for negative values that round to zero)."""
    v = np.asarray(v, np.float32)
    a = np.abs(v).astype(np.float64)
    # index of the nearest grid value; a tie goes to the even code (codes 0, 2, 4, 6 have an
    # even mantissa bit: 0, 1, 2, 4)
    d = np.abs(a[..., None] - E2M1_VALUES)
    best = d.min(axis=-1, keepdims=True)
    near = d == best
    idx = np.where(near.sum(-1) > 1, np.argmax(near & (np.arange(8) % 2 == 0), axis=-1), np.argmin(d, axis=-1))
    idx = np.where(a > 6.0, 7, idx)
    out = E2M1_VALUES[idx].astype(np.float32)
    return np.where(np.signbit(v), -out, out).astype(np.float32)


def e2m1_bits(q):
    """4-bit codes (sign << 3 | index) of E2M1 grid values."""
    q = np.asarray(q, np.float32)
    idx = np.searchsorted(E2M1_VALUES, np.abs(q).astype(np.float64))
    assert np.all(E2M1_VALUES[np.minimum(idx, 7)] == np.abs(q)), "not on the E2M1 grid"
    return (idx | (np.signbit(q).astype(np.int64) << 3)).astype(np.uint8)


def tensor_scale(X):
    """S = amax / (6 * 448) in fp32 (1 for an all-zero tensor)."""
    X = np.asarray(X, np.float32)
    amax = np.float32(np.abs(X).max()) if X.size else np.float32(0)
    return np.float32(amax / np.float32(6 * 448)) if amax > 0 else np.float32(1.0)


def quantize_rows(X, S):
    """Rows X [R, K] (fp32 values) of a tensor whose scale is S: (q [R, K], s [R, K/16])."""
    X = np.asarray(X, np.float32)
    R, K = X.shape
    assert K % BLOCK == 0
    S = np.float32(S)
    blocks = X.reshape(R, K // BLOCK, BLOCK)
    amax_b = np.abs(blocks).max(axis=-1).astype(np.float32)
    six_s = np.float32(np.float32(6) * S)
    s = e4m3_rne(np.minimum((amax_b / six_s).astype(np.float32), np.float32(448)))
    denom = (s * S).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.where(denom > 0, np.float32(1) / denom, np.float32(0)).astype(np.float32)
    v = (blocks * inv[..., None]).astype(np.float32)
    q = e2m1_rne(v)
    return q.reshape(R, K), s.astype(np.float32)


def quantize(X):
    """X [R, K] (fp32 values), K a multiple of 16: (q [R, K] E2M1 values, s [R, K/16] E4M3 values,
    S fp32 tensor scale)."""
    S = tensor_scale(X)
    q, s = quantize_rows(X, S)
    return q, s, S


def dequantize(q, s, S):
    """fp64 values q * s_b * S of a quantized tensor."""
    R, K = q.shape
    return (q.astype(np.float64).reshape(R, K // BLOCK, BLOCK) * s.astype(np.float64)[..., None]).reshape(R, K) \
        * np.float64(S)


def gemm(qa, sa, Sa, qw, sw, Sw, bias=None):
    """Y [M, N] in fp64: S_A * S_W * sum_k (q_A s_A)(q_W s_W) + bias[n] (before the bf16 rounding)."""
    A = dequantize(qa, sa, 1.0)
    W = dequantize(qw, sw, 1.0)
    Y = (A @ W.T) * (np.float64(Sa) * np.float64(Sw))
    if bias is not None:
        Y = Y + np.asarray(bias, np.float64)[None, :]
    return Y


def gemm_abs(qa, sa, qw, sw, Sa, Sw):
    """S_A * S_W * sum_k |q_A s_A||q_W s_W|: the scale of the fp32 accumulation error."""
    A = np.abs(dequantize(qa, sa, 1.0))
    W = np.abs(dequantize(qw, sw, 1.0))
    return (A @ W.T) * (np.float64(Sa) * np.float64(Sw))
