"""Measured properties of the matrix-core instructions the quantized paths rest on.

The all-FP8 attention mode computes its scores with the scaled FP8 MFMA, which sums each group
of 64 products in a fixed-point alignment of its own instead of exactly. The error bound the
FP8-mode parity tests use (tests/sa_checks.FP8_SCORE_REL_ERR: 2^-10 of the sum of |products|
per score) rests on the size of that error, measured here through the library's FP8 debug
tile (the attention kernel's own score code) against exact fp64 sums of the same E4M3 values.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from tests import sa_checks as chk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import dynamic_block_sparse_mean_amd as m

    m.lib()
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _tiles(sa, q, k, bq, bk, picks):
    """FP8-mode score tiles from the GPU and the exact sums of the same E4M3 operands."""
    qd = torch.from_numpy(q).cuda().to(torch.bfloat16)
    kd = torch.from_numpy(k).cuda().to(torch.bfloat16)
    B, H, L, D = q.shape
    ws = sa.prepare(qd, kd, kd, bq, bk, "fp8")
    nK = -(-L // bk)
    plan = torch.arange(nK, dtype=torch.int32, device="cuda").expand(B, H, -(-L // bq), nK).contiguous()
    qv, kv = qd.float().cpu().numpy(), kd.float().cpu().numpy()
    Qh, sq = oracle.quantize_fp8_blocks(qv, bq)
    Kh, sk = oracle.quantize_fp8_blocks(kv, bk)
    Qd, Kd = oracle.dequantize_blocks(Qh, sq, bq), oracle.dequantize_blocks(Kh, sk, bk)
    for (b, h, i, j) in picks:
        got = sa.debug_qk_tile_fp8(ws, (B, H, L, D), bq, bk, plan, b, h, i, j).cpu().numpy().astype(np.float64)
        qi = Qd[b, h, i * bq:(i + 1) * bq]
        kj = Kd[b, h, j * bk:(j + 1) * bk]
        prod = np.abs(qi[:, None, :] * kj[None, :, :])  # [bq, bk, d]
        yield got, qi @ kj.T, prod


def test_fp8_mfma_score_sums_within_the_stated_error(sa):
    """Magnitudes log-uniform over 2^-8..2^8 with random signs (products spread far more than
    the alignment keeps): every score within 2 x 2^-11 of its largest product (two 64-term
    groups per score) and within FP8_SCORE_REL_ERR of the sum of |products|."""
    r = np.random.default_rng(41)
    B, H, L, D, bq, bk = 1, 2, 512, 128, 128, 64
    def draw():
        return (np.exp2(r.uniform(-8, 8, (B, H, L, D))) * r.choice([-1.0, 1.0], (B, H, L, D))).astype(np.float32)
    q, k = draw(), draw()
    worst_max, worst_sum, inexact = 0.0, 0.0, 0
    for got, want, prod in _tiles(sa, q, k, bq, bk, [(0, 0, 0, 0), (0, 1, 3, 7), (0, 0, 2, 5), (0, 1, 1, 2)]):
        err = np.abs(got - want)
        worst_max = max(worst_max, float((err / prod.max(axis=2)).max()))
        worst_sum = max(worst_sum, float((err / prod.sum(axis=2)).max()))
        inexact += int((err > 0).sum())
    say(f"  FP8 MFMA scores: worst error {worst_max:.3e} of the largest product "
        f"(2^{np.log2(worst_max):.2f}), {worst_sum:.3e} of the sum of |products|; {inexact} inexact of {4 * bq * bk}")
    assert inexact > 0  # the spread does reach the alignment (otherwise the test shows nothing)
    assert worst_max <= 2 * 2.0 ** -11
    assert worst_sum <= chk.FP8_SCORE_REL_ERR


def test_fp8_mfma_score_sums_exact_within_four_binades(sa):
    """Codes in [128, 448] (products within four binades): the sums are exact."""
    r = np.random.default_rng(42)
    B, H, L, D, bq, bk = 1, 1, 256, 128, 64, 64
    grid = np.array([v for v in oracle.e4m3_decode(np.arange(256, dtype=np.uint8)) if 128 <= v <= 448])
    def draw():
        x = r.choice(grid, size=(B, H, L, D)) * r.choice([-1.0, 1.0], size=(B, H, L, D))
        x[..., ::64, 0] = 448.0
        return (x / 64.0).astype(np.float32)
    q, k = draw(), draw()
    for got, want, _ in _tiles(sa, q, k, bq, bk, [(0, 0, 0, 0), (0, 0, 3, 1), (0, 0, 1, 2)]):
        assert np.array_equal(got, want)
