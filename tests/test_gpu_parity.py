"""Parity of the HIP path with the CPU oracle, element by element, on seeded inputs.

Bars: pooled means bit-exact (bf16 inputs) or to 1e-14 (fp32); plans exact except rows
excused by the near-tie band; INT8/FP8 operands and scales bit-exact; int32 QK^T tiles
exact; INT8/FP8 attention within rel-L2 5e-3 of the tile-by-tile quantized oracle and, element
by element, within the derived bound of exact attention over the dequantized operands (with
its RMS distance near the predicted one); bf16 attention within max-abs 2e-2 and rel-L2 1e-2 of
exact attention. Outputs are compared on the GPU's own plan, after the plan has been checked
on its own.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, GridConfig, make_qkv
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


def to_dev(x, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype)


def bf16_values(x):
    """float32 numpy array holding the bf16 (RNE) rounding of x, as the GPU sees it."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).float().numpy()


def small_cfg(name, grid, bq, bk, keeps=(0.25,), B=1, H=2, sigma=0.5, seed=11):
    return GridConfig(name, B, H, grid, 128, bq, bk, keeps, (sigma,), "bf16", "int8fp8", seed)


# Shapes spanning several tiles with ragged tails in both block sizes.
SMALL = [
    small_cfg("L1000_q128_k64", (10, 10, 10), 128, 64, (0.2,)),
    small_cfg("L777_q64_k128", (7, 111, 1), 64, 128, (0.3,)),
    small_cfg("L1024_q64_k64", (4, 16, 16), 64, 64, (0.25,)),
    small_cfg("L50_single_block", (2, 5, 5), 128, 64, (0.5,)),
    small_cfg("L1500_q128_k128_B2", (6, 10, 25), 128, 128, (0.34,), B=2, H=2),
]


# ---------------------------------------------------------------- pool
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("L,block", [(1000, 64), (1000, 128), (50, 64), (4096, 128)])
def test_pool_parity(sa, dtype, L, block):
    say(f"pool L={L} block={block} {dtype}")
    x = np.random.default_rng(L + block).standard_normal((2, 3, L, 128)).astype(np.float32) * 3
    xd = to_dev(x, dtype)
    got = sa.pool(xd, block).cpu().numpy()
    want = oracle.pool_block_means(xd.float().cpu().numpy(), block)
    if dtype == torch.bfloat16:
        assert np.array_equal(got, want)
    else:
        np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-15)


def test_pool_strided_blhd(sa):
    x = np.random.default_rng(5).standard_normal((2, 700, 3, 128)).astype(np.float32)
    xd = to_dev(x).transpose(1, 2)  # logical [B, H, L, D] over [B, L, H, D] storage
    got = sa.pool(xd, 64).cpu().numpy()
    want = oracle.pool_block_means(xd.float().cpu().numpy(), 64)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- select
def test_select_exact_from_oracle_means(sa):
    # Same fp64 means on both sides: the GPU top-k must equal the oracle's exactly,
    # including forced ties (duplicated key blocks) and a row of all-equal scores.
    r = np.random.default_rng(3)
    qm = r.standard_normal((1, 3, 20, 128))
    km = r.standard_normal((1, 3, 150, 128))
    km[0, 0, 10] = km[0, 0, 20] = km[0, 0, 30] = km[0, 0, 5]  # ties
    km[0, 1, :] = km[0, 1, 7]  # whole head of equal scores
    qm[0, 2, 3] = 0.0  # a row of zero scores
    km[0, 2, ::3] *= 1e-12  # clusters far apart in magnitude
    for nk in (1, 7, 15, 75, 150):
        got = sa.select(to_dev(qm, torch.float64), to_dev(km, torch.float64), nk).cpu().numpy()
        want = oracle.select_top_blocks(oracle.block_scores(qm, km), nk)
        assert np.array_equal(got, want), nk


@pytest.mark.parametrize("nK", [64, 513, 1500, 2048, 4096])
def test_select_every_row_width(sa, nK):
    # Row widths that use each of the kernel's slot counts (up to the 4096-block limit),
    # with duplicated key blocks so that ties straddle the cut.
    r = np.random.default_rng(nK)
    qm = r.standard_normal((1, 2, 6, 128))
    km = r.standard_normal((1, 2, nK, 128))
    km[0, 0, 1::5] = km[0, 0, 0]
    km[0, 1, nK // 2:] = km[0, 1, : nK - nK // 2]
    for nk in sorted({1, max(1, nK // 10), nK // 2, nK - 1, nK} - {0}):
        got = sa.select(to_dev(qm, torch.float64), to_dev(km, torch.float64), nk).cpu().numpy()
        want = oracle.select_top_blocks(oracle.block_scores(qm, km), nk)
        assert np.array_equal(got, want), nk


def test_select_geometric_scores_use_the_byte_passes(sa):
    # Scores 2^j spread over a huge range defeat the value histogram (each pass removes
    # one block); the byte-wise passes must still resolve the row exactly.
    nK = 1200
    km = np.zeros((1, 1, nK, 128))
    km[0, 0, :, 0] = 2.0 ** (np.arange(nK) % 900 - 450)
    qm = np.zeros((1, 1, 4, 128))
    qm[0, 0, :, 0] = [1.0, -1.0, 3.0, 1e-300]
    for nk in (1, 60, 600, 1199):
        got = sa.select(to_dev(qm, torch.float64), to_dev(km, torch.float64), nk).cpu().numpy()
        want = oracle.select_top_blocks(oracle.block_scores(qm, km), nk)
        assert np.array_equal(got, want), nk


# ---------------------------------------------------------------- plan
def _plan_case(sa, cfg, keep, fp32=False):
    q, k, _ = make_qkv(cfg)
    dt = torch.float32 if fp32 else torch.bfloat16
    qd, kd = to_dev(q, dt), to_dev(k, dt)
    gp = sa.plan(qd, kd, cfg.block_q, cfg.block_k, keep).cpu().numpy()
    qv, kv = qd.float().cpu().numpy(), kd.float().cpu().numpy()
    S, mag = chk.pooled_scores(qv, kv, cfg.block_q, cfg.block_k)
    nk = oracle.n_keep(S.shape[-1], keep)
    return gp, (S, mag), nk


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_plan_parity_small(sa, cfg):
    say(f"plan {cfg.name}")
    gp, (S, mag), nk = _plan_case(sa, cfg, cfg.keep)
    excused = chk.compare_plan(gp, S, nk, mag)
    assert excused <= 1


def test_plan_parity_tiny_fp32(sa):
    cfg = CONFIGS["tiny"]
    gp, (S, mag), nk = _plan_case(sa, cfg, cfg.keep, fp32=True)
    assert nk == 4
    assert chk.compare_plan(gp, S, nk, mag) == 0


def test_plan_keep_one_is_every_block(sa):
    cfg = SMALL[0]
    gp, (S, _), nk = _plan_case(sa, cfg, 1.0)
    assert nk == S.shape[-1]
    assert np.array_equal(gp, np.broadcast_to(np.arange(nk, dtype=np.int32), gp.shape))


# ---------------------------------------------------------------- plan + prepare in one pass
@pytest.mark.parametrize("mode", ["int8fp8", "fp8", "bf16"])
@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_plan_prepare_equals_plan_then_prepare(sa, cfg, mode):
    say(f"plan_prepare {cfg.name} {mode}")
    q, k, v = make_qkv(cfg)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    B, H, L, _ = q.shape
    p1 = sa.plan(qd, kd, cfg.block_q, cfg.block_k, cfg.keep)
    ws1 = sa.prepare(qd, kd, vd, cfg.block_q, cfg.block_k, mode)
    p2, ws2 = sa.plan_prepare(qd, kd, vd, cfg.block_q, cfg.block_k, cfg.keep, mode)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2)
    lay = sa.forward_layout(B, H, L, 128, cfg.block_q, cfg.block_k, mode)
    a = chk.workspace_pieces(ws1.cpu().numpy(), lay, B, H, cfg.block_q, cfg.block_k, mode)
    b = chk.workspace_pieces(ws2.cpu().numpy(), lay, B, H, cfg.block_q, cfg.block_k, mode)
    for name in a:
        assert np.array_equal(a[name], b[name]), name


# ---------------------------------------------------------------- quantize
@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_quantize_bit_exact(sa, cfg):
    say(f"quantize {cfg.name}")
    q, k, v = make_qkv(cfg)
    q[0, 0, : min(cfg.block_q, cfg.L)] = 0.0  # an all-zero Q block
    v[0, -1, -5:] = 0.0
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    B, H, L, _ = q.shape
    ws = sa.prepare(qd, kd, vd, cfg.block_q, cfg.block_k, "int8fp8")
    torch.cuda.synchronize()
    wsn = ws.cpu().numpy()
    lay = sa.forward_layout(B, H, L, 128, cfg.block_q, cfg.block_k, "int8fp8")
    qv, kv, vv = (bf16_values(x) for x in (q, k, v))
    Qh, sq = oracle.quantize_int8_blocks(qv, cfg.block_q)
    Kh, sk = oracle.quantize_int8_blocks(kv, cfg.block_k)
    Vq, sv = oracle.quantize_fp8_blocks(vv, cfg.block_k)
    gq, gq_pad = chk.decode_q_int8(wsn, lay, B, H, L, cfg.block_q)
    gk, gk_pad = chk.decode_k(wsn, lay, B, H, L, cfg.block_k)
    gv, gv_pad = chk.decode_vt_fp8(wsn, lay, B, H, L, cfg.block_k)
    gsq, gsk, gsv = chk.scales(wsn, lay, B, H)
    assert np.array_equal(gsq, sq) and np.array_equal(gsk, sk) and np.array_equal(gsv, sv)
    assert np.array_equal(gq, Qh)
    assert np.array_equal(gk.view(np.int8), Kh)
    assert np.array_equal(gv, oracle.e4m3_bits(Vq))
    assert not gq_pad.any() and not gk_pad.any() and not gv_pad.any()


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_quantize_fp8_mode_bit_exact(sa, cfg):
    # All-FP8 mode: Q and K are E4M3 codes (power-of-two block scales) in the INT8 layout.
    say(f"quantize fp8 {cfg.name}")
    q, k, v = make_qkv(cfg)
    q[0, 0, : min(cfg.block_q, cfg.L)] = 0.0  # an all-zero Q block
    k[0, -1, -3:] *= 1e6  # a block whose scale is set by a few large values
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    B, H, L, _ = q.shape
    ws = sa.prepare(qd, kd, vd, cfg.block_q, cfg.block_k, "fp8")
    torch.cuda.synchronize()
    wsn = ws.cpu().numpy()
    lay = sa.forward_layout(B, H, L, 128, cfg.block_q, cfg.block_k, "fp8")
    qv, kv, vv = (bf16_values(x) for x in (q, k, v))
    Qh, sq = oracle.quantize_fp8_blocks(qv, cfg.block_q)
    Kh, sk = oracle.quantize_fp8_blocks(kv, cfg.block_k)
    Vq, sv = oracle.quantize_fp8_blocks(vv, cfg.block_k)
    gq, gq_pad = chk.decode_q_int8(wsn, lay, B, H, L, cfg.block_q)
    gk, gk_pad = chk.decode_k(wsn, lay, B, H, L, cfg.block_k)
    gv, gv_pad = chk.decode_vt_fp8(wsn, lay, B, H, L, cfg.block_k)
    gsq, gsk, gsv = chk.scales(wsn, lay, B, H)
    assert np.array_equal(gsq, sq) and np.array_equal(gsk, sk) and np.array_equal(gsv, sv)
    assert np.array_equal(gq.view(np.uint8), oracle.e4m3_bits(Qh))
    assert np.array_equal(gk.view(np.uint8), oracle.e4m3_bits(Kh))
    assert np.array_equal(gv, oracle.e4m3_bits(Vq))
    assert not gq_pad.any() and not gk_pad.any() and not gv_pad.any()


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_attend_fp8_mode_parity(sa, cfg):
    say(f"attend fp8 {cfg.name}")
    (qv, kv, vv), pn, got = _attend_case(sa, cfg, "fp8")
    Qh, sq = oracle.quantize_fp8_blocks(qv, cfg.block_q)
    Kh, sk = oracle.quantize_fp8_blocks(kv, cfg.block_k)
    Vq, sv = oracle.quantize_fp8_blocks(vv, cfg.block_k)
    # the FP8 MFMA's score sums (tests/test_gpu_hw.py) enter the bound against exact attention
    r = chk.check_quantized(got, Qh, sq, Kh, sk, Vq, sv, pn, cfg.block_q, cfg.block_k, qk_fp8=True)
    say("  " + chk.fmt(r))


@pytest.mark.parametrize("cfg", [SMALL[0], SMALL[1], SMALL[4]], ids=lambda c: c.name)
def test_attend_fp8_mode_exact_sums(sa, cfg):
    # Q and K whose E4M3 codes all lie in [128, 448] (one code of 448 per block pins the
    # power-of-two scale at 1): every product lies in [2^14, 448^2], within four binades,
    # so the FP8 MFMA sums them exactly, and the FP8 mode must then match the oracle as
    # closely as the INT8 mode does (this checks the operand pairing and both scales).
    say(f"attend fp8 exact sums {cfg.name}")
    r = np.random.default_rng(cfg.L)
    B, H, L = cfg.B, cfg.H, cfg.L
    grid = np.array([v for v in oracle.e4m3_decode(np.arange(256, dtype=np.uint8)) if 128 <= v <= 448])
    def draw():
        x = r.choice(grid, size=(B, H, L, 128)) * r.choice([-1.0, 1.0], size=(B, H, L, 128))
        x[..., ::64, 0] = 448.0  # every 64-row block holds the largest code
        return (x / 64.0).astype(np.float32)  # block scale 2^-6; logits stay moderate
    q, k = draw(), draw()
    v = r.standard_normal((B, H, L, 128)).astype(np.float32)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    p = sa.plan(qd, kd, cfg.block_q, cfg.block_k, cfg.keep)
    got = sa.forward(qd, kd, vd, p, cfg.block_q, cfg.block_k, "fp8", sm_scale=1.0 / 256).float().cpu().numpy()
    pn = p.cpu().numpy()
    qv, kv, vv = (bf16_values(x) for x in (q, k, v))
    Qh, sq = oracle.quantize_fp8_blocks(qv, cfg.block_q)
    Kh, sk = oracle.quantize_fp8_blocks(kv, cfg.block_k)
    Vq, sv = oracle.quantize_fp8_blocks(vv, cfg.block_k)
    assert np.all(np.isin(np.abs(Qh), np.concatenate([[0.0], grid])))  # codes stayed in range
    # exact sums: held to the INT8 mode's checks, the RMS one included
    r = chk.check_quantized(got, Qh, sq, Kh, sk, Vq, sv, pn, cfg.block_q, cfg.block_k, sm=1.0 / 256)
    say("  " + chk.fmt(r))


# ---------------------------------------------------------------- int32 QK^T tiles
@pytest.mark.parametrize("cfg", [SMALL[0], SMALL[1], SMALL[4]], ids=lambda c: c.name)
def test_debug_qk_tile_exact(sa, cfg):
    say(f"qk tile {cfg.name}")
    q, k, v = make_qkv(cfg)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    B, H, L, _ = q.shape
    p = sa.plan(qd, kd, cfg.block_q, cfg.block_k, cfg.keep)
    ws = sa.prepare(qd, kd, vd, cfg.block_q, cfg.block_k, "int8fp8")
    pn = p.cpu().numpy()
    Qh, _ = oracle.quantize_int8_blocks(bf16_values(q), cfg.block_q)
    Kh, _ = oracle.quantize_int8_blocks(bf16_values(k), cfg.block_k)
    nQ = pn.shape[2]
    for (b, h, i, t) in [(0, 0, 0, 0), (B - 1, H - 1, nQ - 1, pn.shape[3] - 1), (0, H - 1, nQ // 2, 0)]:
        tile = sa.debug_qk_tile(ws, (B, H, L, 128), cfg.block_q, cfg.block_k, p, b, h, i, t).cpu().numpy()
        j = int(pn[b, h, i, t])
        r0, r1 = i * cfg.block_q, min((i + 1) * cfg.block_q, L)
        c0, c1 = j * cfg.block_k, min((j + 1) * cfg.block_k, L)
        want = Qh[b, h, r0:r1].astype(np.int64) @ Kh[b, h, c0:c1].astype(np.int64).T
        assert np.array_equal(tile[: r1 - r0, : c1 - c0].astype(np.int64), want), (b, h, i, t)
        assert not tile[r1 - r0:].any() and not tile[:, c1 - c0:].any()


# ---------------------------------------------------------------- attention
def _attend_case(sa, cfg, mode, keep=None):
    keep = cfg.keep if keep is None else keep
    q, k, v = make_qkv(cfg)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    p = sa.plan(qd, kd, cfg.block_q, cfg.block_k, keep)
    out = sa.forward(qd, kd, vd, p, cfg.block_q, cfg.block_k, mode)
    torch.cuda.synchronize()
    return (bf16_values(q), bf16_values(k), bf16_values(v)), p.cpu().numpy(), out.float().cpu().numpy()


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_attend_int8fp8_parity(sa, cfg):
    say(f"attend int8fp8 {cfg.name}")
    (qv, kv, vv), pn, got = _attend_case(sa, cfg, "int8fp8")
    Qh, sq = oracle.quantize_int8_blocks(qv, cfg.block_q)
    Kh, sk = oracle.quantize_int8_blocks(kv, cfg.block_k)
    Vq, sv = oracle.quantize_fp8_blocks(vv, cfg.block_k)
    r = chk.check_quantized(got, Qh, sq, Kh, sk, Vq, sv, pn, cfg.block_q, cfg.block_k)
    say("  " + chk.fmt(r))


@pytest.mark.parametrize("mode", ["int8fp8", "fp8", "bf16"])
def test_attend_constant_v_gives_the_constant(sa, mode):
    """Weights that sum to one: with V constant over each head (0.75 and -3, both exact in bf16
    and, after the block scale, in E4M3), every output is that constant. In the quantized modes
    the numerator sum_k p^_k v and the row sum sum_k p^_k come from two FP8 MFMAs over the same
    weights, each within 2^-10.9 of a tile's largest weight per 64-term sum, so the ratio is
    within 2^-9.5 of v before the bf16 rounding (2^-9): 2^-8 bounds both."""
    cfg = SMALL[0]  # L = 1000 (ragged in both block sizes), H = 2
    q, k, v = make_qkv(cfg)
    v = np.empty_like(v)
    v[:, 0], v[:, 1] = 0.75, -3.0
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    p = sa.plan(qd, kd, cfg.block_q, cfg.block_k, cfg.keep)
    out = sa.forward(qd, kd, vd, p, cfg.block_q, cfg.block_k, mode).float().cpu().numpy()
    rel = np.abs(out / v - 1.0).max()
    say(f"constant V {mode}: worst |out / v - 1| = {rel:.3e}")
    assert rel <= 2.0 ** -8


@pytest.mark.parametrize("cfg", [CONFIGS["tiny"]] + SMALL, ids=lambda c: c.name)
def test_attend_bf16_parity(sa, cfg):
    say(f"attend bf16 {cfg.name}")
    (qv, kv, vv), pn, got = _attend_case(sa, cfg, "bf16")
    want = oracle.attend_exact(qv, kv, vv, pn, cfg.block_q, cfg.block_k)
    err, mx = chk.rel_l2(got, want), np.abs(got - want).max()
    say(f"  rel-L2 {err:.2e} max-abs {mx:.2e}")
    assert err <= 1e-2 and mx <= 2e-2


def test_attend_keep_one_is_dense_attention(sa):
    cfg = SMALL[0]
    (qv, kv, vv), pn, got = _attend_case(sa, cfg, "bf16", keep=1.0)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qv).double(), torch.from_numpy(kv).double(), torch.from_numpy(vv).double()).numpy()
    assert chk.rel_l2(got, want) <= 1e-2 and np.abs(got - want).max() <= 2e-2


@pytest.mark.parametrize("mode", ["int8fp8", "fp8", "bf16"])
def test_attend_zero_blocks(sa, mode):
    """All-zero blocks through the attention: a zero Q block (scale 0: every score of its rows
    is 0, so they average V uniformly over the kept keys), a zero K block and a zero V block
    (scale 0 and E8M0 exponent 0), on a ragged shape; the plan is the library's, with the zero
    key block forced into every row so that its tiles are visited."""
    cfg = SMALL[0]  # L = 1000, block_q 128, block_k 64, H = 2
    bq, bk, keep = cfg.block_q, cfg.block_k, 0.3
    q, k, v = make_qkv(cfg)
    q, k, v = q.copy(), k.copy(), v.copy()
    q[:, 0, bq:2 * bq] = 0.0
    k[:, 1, 3 * bk:4 * bk] = 0.0
    v[:, :, 5 * bk:6 * bk] = 0.0
    say(f"zero blocks {mode}: {cfg.name} keep={keep}")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    p = sa.plan(qd, kd, bq, bk, keep)
    pn = p.cpu().numpy().copy()
    for zero_blk in (3, 5):  # make every row keep key blocks 3 and 5 (replacing its first entries)
        has = (pn == zero_blk).any(axis=3, keepdims=True)
        col = 0 if zero_blk == 3 else 1
        pn[..., col:col + 1] = np.where(has, pn[..., col:col + 1], zero_blk)
    pn = np.sort(pn, axis=3)
    assert all(len(set(r)) == len(r) for r in pn.reshape(-1, pn.shape[3]).tolist())
    assert (pn == 3).any(axis=3).all() and (pn == 5).any(axis=3).all()
    p.copy_(torch.from_numpy(pn))
    out = sa.forward(qd, kd, vd, p, bq, bk, mode)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    qv, kv, vv = bf16_values(q), bf16_values(k), bf16_values(v)
    assert np.isfinite(got).all()
    if mode == "bf16":
        want = oracle.attend_exact(qv, kv, vv, pn, bq, bk)
        err, mx = chk.rel_l2(got, want), np.abs(got - want).max()
        say(f"  rel-L2 vs exact {err:.2e}, max-abs {mx:.2e}")
        assert err <= 1e-2 and mx <= 2e-2
        return
    quant = oracle.quantize_int8_blocks if mode == "int8fp8" else oracle.quantize_fp8_blocks
    Qh, sq = quant(qv, bq)
    Kh, sk = quant(kv, bk)
    Vq, sv = oracle.quantize_fp8_blocks(vv, bk)
    assert not Qh[0, 0, bq:2 * bq].any() and not Kh[0, 1, 3 * bk:4 * bk].any()
    assert not Vq[:, :, 5 * bk:6 * bk].any()
    r = chk.check_quantized(got, Qh, sq, Kh, sk, Vq, sv, pn, bq, bk, qk_fp8=mode == "fp8")
    say("  " + chk.fmt(r))


@pytest.mark.parametrize("mode", ["int8fp8", "fp8", "bf16"])
def test_attend_far_rescale(sa, mode):
    """Every row's running maximum rises by far more than 64 binades after its first tile:
    the last key block holds keys 40 times larger than the others (all rows share a mean
    direction), so the plan keeps it last, after blocks whose scores are ~150 log2 units lower.
    The quantized kernels bring their accumulators to the new reference by an exact power of
    two there; the bf16 kernel's lazy rescale takes the same step."""
    B, H, L, d, bq, bk, keep = 1, 1, 1024, 128, 128, 64, 0.25
    rng = np.random.default_rng(5)
    u = np.full(d, 0.5)
    q = (u + 0.3 * rng.standard_normal((B, H, L, d))).astype(np.float32)
    k = (u + 0.3 * rng.standard_normal((B, H, L, d))).astype(np.float32)
    k[:, :, L - bk:] *= 40.0
    v = rng.standard_normal((B, H, L, d)).astype(np.float32)
    say(f"far rescale {mode}: L={L} bq={bq} bk={bk} keep={keep}")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    p = sa.plan(qd, kd, bq, bk, keep)
    out = sa.forward(qd, kd, vd, p, bq, bk, mode)
    torch.cuda.synchronize()
    pn, got = p.cpu().numpy(), out.float().cpu().numpy()
    qv, kv, vv = bf16_values(q), bf16_values(k), bf16_values(v)
    # the precondition: the last key block is kept, last, and every row's exact scores there
    # exceed those of its first kept block by more than 64 (log2 units) plus a wide margin
    nK = L // bk
    lg = (qv[0, 0].astype(np.float64) @ kv[0, 0].astype(np.float64).T) / math.sqrt(d) * oracle.LOG2E
    for i in range(L // bq):
        kept = sorted(int(j) for j in pn[0, 0, i])
        assert kept[-1] == nK - 1 and len(kept) >= 2
        rows = lg[i * bq:(i + 1) * bq]
        first = rows[:, kept[0] * bk:(kept[0] + 1) * bk].max(axis=1)
        last = rows[:, (nK - 1) * bk:].max(axis=1)
        assert (last - first).min() > 100.0
    if mode == "bf16":
        want = oracle.attend_exact(qv, kv, vv, pn, bq, bk)
        err, mx = chk.rel_l2(got, want), np.abs(got - want).max()
        say(f"  rel-L2 vs exact {err:.2e}, max-abs {mx:.2e}")
        assert err <= 1e-2 and mx <= 2e-2
        return
    quant = oracle.quantize_int8_blocks if mode == "int8fp8" else oracle.quantize_fp8_blocks
    Qh, sq = quant(qv, bq)
    Kh, sk = quant(kv, bk)
    Vq, sv = oracle.quantize_fp8_blocks(vv, bk)
    r = chk.check_quantized(got, Qh, sq, Kh, sk, Vq, sv, pn, bq, bk, qk_fp8=mode == "fp8")
    say("  " + chk.fmt(r))


def test_forward_is_prepare_then_attend_and_deterministic(sa):
    cfg = SMALL[0]
    q, k, v = make_qkv(cfg)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    p = sa.plan(qd, kd, cfg.block_q, cfg.block_k, cfg.keep)
    p2 = sa.plan(qd, kd, cfg.block_q, cfg.block_k, cfg.keep)
    assert torch.equal(p, p2)
    for mode in ("int8fp8", "bf16"):
        a = sa.forward(qd, kd, vd, p, cfg.block_q, cfg.block_k, mode)
        b = sa.forward(qd, kd, vd, p, cfg.block_q, cfg.block_k, mode)
        ws = sa.prepare(qd, kd, vd, cfg.block_q, cfg.block_k, mode)
        c = sa.attend(qd, p, ws, cfg.block_q, cfg.block_k, mode)
        assert torch.equal(a, b) and torch.equal(a, c), mode


def test_strided_blhd_inputs_match(sa):
    cfg = SMALL[0]
    q, k, v = make_qkv(cfg)
    dense = [to_dev(x) for x in (q, k, v)]
    strided = [to_dev(np.swapaxes(x, 1, 2)).transpose(1, 2) for x in (q, k, v)]
    assert strided[0].stride(2) != 128
    p1 = sa.plan(dense[0], dense[1], cfg.block_q, cfg.block_k, cfg.keep)
    p2 = sa.plan(strided[0], strided[1], cfg.block_q, cfg.block_k, cfg.keep)
    assert torch.equal(p1, p2)
    for mode in ("int8fp8", "bf16"):
        o1 = sa.forward(*dense, p1, cfg.block_q, cfg.block_k, mode)
        o2 = sa.forward(*strided, p1, cfg.block_q, cfg.block_k, mode,
                        out=torch.empty_like(strided[0]))
        assert torch.equal(o1, o2.contiguous()), mode


def test_out_of_range_plan_entries_are_skipped(sa):
    cfg = SMALL[2]
    q, k, v = make_qkv(cfg)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    p = sa.plan(qd, kd, cfg.block_q, cfg.block_k, cfg.keep)
    bad = p.clone()
    bad[..., -1] = 10 ** 6  # the last kept block of every row is invalid
    for mode in ("int8fp8", "bf16"):
        o_bad = sa.forward(qd, kd, vd, bad, cfg.block_q, cfg.block_k, mode)
        o_ref = sa.forward(qd, kd, vd, p[..., :-1].contiguous(), cfg.block_q, cfg.block_k, mode)
        assert torch.equal(o_bad, o_ref), mode


# ---------------------------------------------------------------- full-size workloads, sampled
@pytest.fixture(scope="module")
def full_720p(sa):
    cfg = CONFIGS["720p"]
    say("generating 720p inputs (B=1 H=40 L=75600)")
    q, k, v = make_qkv(cfg)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    del q, k, v
    p = sa.plan(qd, kd, cfg.block_q, cfg.block_k, cfg.keep)
    out = sa.forward(qd, kd, vd, p, cfg.block_q, cfg.block_k, "int8fp8")
    torch.cuda.synchronize()
    return cfg, (qd, kd, vd), p, out


def test_720p_plan_prepare_is_plan_then_prepare(sa, full_720p):
    cfg, (qd, kd, vd), p, _ = full_720p
    p2, ws2 = sa.plan_prepare(qd, kd, vd, cfg.block_q, cfg.block_k, cfg.keep, "int8fp8")
    ws1 = sa.prepare(qd, kd, vd, cfg.block_q, cfg.block_k, "int8fp8")
    torch.cuda.synchronize()
    assert torch.equal(p, p2)
    lay = sa.forward_layout(1, 40, cfg.L, 128, cfg.block_q, cfg.block_k, "int8fp8")
    for name in ("q_off", "k_off", "v_off", "sq_off", "sk_off", "sv_off"):
        n = {"q_off": 40 * lay["nQ"] * 128 * 128, "k_off": 40 * lay["nK"] * 64 * 128,
             "v_off": 40 * lay["nK"] * 64 * 128, "sq_off": 40 * lay["nQ"] * 4,
             "sk_off": 40 * lay["nK"] * 4, "sv_off": 40 * lay["nK"] * 4}[name]
        assert torch.equal(ws1[lay[name]: lay[name] + n], ws2[lay[name]: lay[name] + n]), name


def test_720p_plan_sampled_heads(sa, full_720p):
    cfg, (qd, kd, _), p, _ = full_720p
    pn = p.cpu().numpy()
    assert pn.shape == (1, 40, 591, 119)
    for h in (0, 17, 39):
        qv = qd[:, h:h + 1].float().cpu().numpy()
        kv = kd[:, h:h + 1].float().cpu().numpy()
        S, mag = chk.pooled_scores(qv, kv, 128, 64)
        excused = chk.compare_plan(pn[:, h:h + 1], S, 119, mag, label=f"head {h} ")
        say(f"  head {h}: {excused} rows excused by the near-tie band")
        assert excused <= 5


def test_720p_attention_sampled_blocks(sa, full_720p):
    cfg, (qd, kd, vd), p, out = full_720p
    pn = p.cpu().numpy()
    for h, i in [(0, 0), (5, 300), (39, 590), (22, 123)]:  # 590 is the short last query block
        sl = lambda x: x[:, h:h + 1].float().cpu().numpy()
        Qh, sq = oracle.quantize_int8_blocks(sl(qd), 128)
        Kh, sk = oracle.quantize_int8_blocks(sl(kd), 64)
        Vq, sv = oracle.quantize_fp8_blocks(sl(vd), 64)
        r0, r1 = 128 * i, min(128 * i + 128, cfg.L)
        got = np.full(Qh.shape, np.nan)
        got[0, 0, r0:r1] = out[0, h, r0:r1].float().cpu().numpy()
        r = chk.check_quantized(got, Qh, sq, Kh, sk, Vq, sv, pn[:, h:h + 1], 128, 64, rows=[(0, 0, i)])
        say(f"  head {h} block {i}: " + chk.fmt(r))
    assert torch.isfinite(out.float()).all()


def test_480p_bf16_sampled_blocks(sa):
    cfg = CONFIGS["480p"]
    say("generating 480p inputs (B=1 H=40 L=32760)")
    q, k, v = make_qkv(cfg)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    del q, k, v
    p = sa.plan(qd, kd, cfg.block_q, cfg.block_k, cfg.keep)
    out = sa.forward(qd, kd, vd, p, cfg.block_q, cfg.block_k, "bf16")
    torch.cuda.synchronize()
    pn = p.cpu().numpy()
    assert pn.shape == (1, 40, 256, 103)
    for h, i in [(0, 0), (13, 255), (39, 100)]:
        sl = lambda x: x[:, h:h + 1].float().cpu().numpy()
        qv, kv, vv = sl(qd), sl(kd), sl(vd)
        r0, r1 = 128 * i, min(128 * i + 128, cfg.L)
        S, mag = chk.pooled_scores(qv, kv, 128, 64)
        chk.compare_plan(pn[:, h:h + 1], S, 103, mag, label=f"head {h} ")
        want = oracle.attend_exact(qv, kv, vv, pn[:, h:h + 1], 128, 64, rows=[(0, 0, i)])[0, 0, r0:r1]
        got = out[0, h, r0:r1].float().cpu().numpy()
        err, mx = chk.rel_l2(got, want), np.abs(got - want).max()
        say(f"  head {h} block {i}: rel-L2 {err:.2e} max-abs {mx:.2e}")
        assert err <= 1e-2 and mx <= 2e-2
