"""NVFP4 quantizer and block-scaled GEMM against the oracle.

Bars: codes, block scales and the tensor scale bit-exact (both sides take every rounding
decision with the same fp32 operations); GEMM outputs within |Y - Y*| <= 2^-8 |Y*| (the bf16
rounding) + K * 2^-24 * S_A S_W sum_k |a_k w_k| (fp32 accumulation of exact products, worst case)
of the oracle's fp64 Y*, and within rel-L2 4e-3 overall; at the 720p FFN shape on sampled outputs.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import nvfp4 as nf
from synth import wide_rows

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import dynamic_block_sparse_mean_amd as m

    m.lib()
    return m


def bf16_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).cuda()


def unpack_codes(codes):
    """uint8 [R, K/2] -> E2M1 values [R, K] (low nibble first)."""
    c = codes.astype(np.uint8)
    nib = np.stack([c & 15, c >> 4], axis=-1).reshape(c.shape[0], -1)
    mag = nf.E2M1_VALUES[nib & 7].astype(np.float32)
    return np.where(nib & 8, -mag, mag).astype(np.float32)


def e4m3_values(b):
    return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn).float().numpy()


def check_quant(sa, X, ld_pad=0):
    R, K = X.shape
    xd = bf16_dev(np.pad(X, ((0, 0), (0, ld_pad))))[:, :K] if ld_pad else bf16_dev(X)
    xv = xd.float().cpu().numpy()
    codes, scales, S = sa.nvfp4_quantize(xd)
    torch.cuda.synchronize()
    q, s, Sw = nf.quantize(xv)
    assert np.float32(S.item()) == Sw, (S.item(), Sw)
    gs = e4m3_values(scales.cpu().numpy())
    assert np.array_equal(gs, s), "block scales"
    gq = unpack_codes(codes.cpu().numpy())
    bad = ~((gq == q) & (np.signbit(gq) == np.signbit(q)))
    assert not bad.any(), f"{bad.sum()} codes differ, first at {np.argwhere(bad)[0]}"
    return codes, scales, S


@pytest.mark.parametrize("R,K,ld_pad", [(1, 64, 0), (37, 128, 0), (300, 640, 8), (64, 5120, 0)])
def test_quantize_bit_exact(sa, R, K, ld_pad):
    say(f"nvfp4 quantize R={R} K={K} ld_pad={ld_pad}")
    X = wide_rows(70 + R, (R, K))
    X[0, :16] = np.linspace(-7, 7, 16)  # every E2M1 step and both saturations in one block
    check_quant(sa, X, ld_pad)


def test_quantize_block_that_separates_reciprocal_from_division(sa):
    """Elements at exact E2M1 midpoints of their block (scale 0.9375, tensor scale 1): the
    library multiplies by the block's fp32 reciprocal, as the oracle does, so they land just
    above the midpoints (1.5, 3, 6), where a per-element division would give 1, 2, 4."""
    X = np.zeros((2, 256), np.float32)
    X[0, :4] = [5.625, 1.171875, 2.34375, 4.6875]
    X[1, 0] = 2688.0
    codes, _, _ = check_quant(sa, X)
    assert np.array_equal(unpack_codes(codes.cpu().numpy())[0, :4], [6.0, 1.5, 3.0, 6.0])


def test_quantize_zero_tensor(sa):
    codes, scales, S = check_quant(sa, np.zeros((3, 64), np.float32))
    assert S.item() == 1.0 and not scales.any() and not codes.any()


def check_gemm(sa, M, N, K, bias=True, seed=0):
    r = np.random.default_rng(seed)
    A = (r.standard_normal((M, K)) * np.exp(r.uniform(-2, 2, (M, 1)))).astype(np.float32)
    W = (r.standard_normal((N, K)) * 0.05).astype(np.float32)
    ad, wd = bf16_dev(A), bf16_dev(W)
    b = bf16_dev(r.standard_normal(N)) if bias else None
    qa = sa.nvfp4_quantize(ad)
    qw = sa.nvfp4_quantize(wd)
    y = sa.nvfp4_gemm(qa, qw, b)
    torch.cuda.synchronize()
    Aq, As, AS = nf.quantize(ad.float().cpu().numpy())
    Wq, Ws, WS = nf.quantize(wd.float().cpu().numpy())
    bv = b.float().cpu().numpy() if bias else None
    want = nf.gemm(Aq, As, AS, Wq, Ws, WS, bv)
    mag = nf.gemm_abs(Aq, As, Wq, Ws, AS, WS)
    got = y.float().cpu().numpy()
    bound = 2.0 ** -8 * np.abs(want) + K * 2.0 ** -24 * mag + 1e-30
    err = np.abs(got - want)
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.2f} at {np.unravel_index(np.argmax(err / bound), err.shape)}"
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    say(f"  rel-L2 {rel:.2e}, max err/bound {np.max(err / bound):.3f}")
    assert rel <= 4e-3


@pytest.mark.parametrize("M,N,K", [(1, 8, 256), (100, 64, 256), (300, 264, 512), (257, 512, 768), (513, 1032, 1024),
                                   (1000, 2056, 2304)])
def test_gemm_parity(sa, M, N, K):
    say(f"nvfp4 gemm M={M} N={N} K={K}")
    check_gemm(sa, M, N, K, bias=True, seed=M + N + K)


def test_gemm_without_bias(sa):
    check_gemm(sa, 256, 256, 256, bias=False, seed=5)


def test_gemm_rejects_k_not_multiple_of_256(sa):
    x = torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda")
    q = sa.nvfp4_quantize(x)
    with pytest.raises(RuntimeError, match="multiple of 256"):
        sa.nvfp4_gemm(q, q)


def test_gemm_720p_ffn_sampled(sa):
    """The 720p FFN up-projection shape (tokens 75600, K = 5120, N = 13824) at full size, in the
    launch configuration the benchmark times; sampled outputs recomputed by the oracle from the
    same bf16 inputs (the tensor scales from the whole tensors, the sampled rows quantized)."""
    M, N, K = 75600, 13824, 5120
    say(f"nvfp4 gemm 720p FFN M={M} N={N} K={K}")
    g = torch.Generator(device="cuda").manual_seed(3)
    ad = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    wd = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    b = (torch.randn(N, generator=g, device="cuda") * 0.1).to(torch.bfloat16)
    qa = sa.nvfp4_quantize(ad)
    qw = sa.nvfp4_quantize(wd)
    y = sa.nvfp4_gemm(qa, qw, b)
    torch.cuda.synchronize()
    SA = nf.tensor_scale(ad.float().cpu().numpy())
    SW = nf.tensor_scale(wd.float().cpu().numpy())
    assert np.float32(qa[2].item()) == SA and np.float32(qw[2].item()) == SW
    r = np.random.default_rng(9)
    ms = np.unique(np.concatenate([[0, M - 1], r.integers(0, M, 14)]))
    ns = np.unique(np.concatenate([[0, N - 1], r.integers(0, N, 14)]))
    Aq, As = nf.quantize_rows(ad[torch.from_numpy(ms).cuda()].float().cpu().numpy(), SA)
    Wq, Ws = nf.quantize_rows(wd[torch.from_numpy(ns).cuda()].float().cpu().numpy(), SW)
    # the sampled rows' codes as the GPU wrote them
    assert np.array_equal(unpack_codes(qa[0][torch.from_numpy(ms).cuda()].cpu().numpy()), Aq)
    assert np.array_equal(unpack_codes(qw[0][torch.from_numpy(ns).cuda()].cpu().numpy()), Wq)
    bv = b.float().cpu().numpy()[ns]
    want = nf.gemm(Aq, As, SA, Wq, Ws, SW, bv)
    mag = nf.gemm_abs(Aq, As, Wq, Ws, SA, SW)
    got = y[torch.from_numpy(ms).cuda()][:, torch.from_numpy(ns).cuda()].float().cpu().numpy()
    bound = 2.0 ** -8 * np.abs(want) + K * 2.0 ** -24 * mag
    err = np.abs(got - want)
    say(f"  {len(ms)}x{len(ns)} outputs: max err/bound {np.max(err / bound):.3f}")
    assert np.all(err <= bound)
