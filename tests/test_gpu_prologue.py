"""The Q/K prologue (RMSNorm, then 3-D RoPE) fused into the plan-and-quantize pass, against the
oracle: block means, the plan, the quantized operands and scales, and the attention output.

Bars: block means within the fp64 summation bound (n - 1) * 2^-53 * mean|x| (the same fp32
values summed in another order); plans exact but for near-tie rows; INT8/FP8 codes and scales
bit-exact (both sides compute the prologue with the same fp32 operations and quantize that); V
untouched by the prologue; attention within the quantized-path bound of the other parity
tests (rel-L2 5e-3 against the tile-by-tile quantized oracle, and within the derived bound of
exact attention over the dequantized operands).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import prologue as po
from synth import CONFIGS, GridConfig, make_qkv
from tests import sa_checks as chk

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


def bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def gains(seed, H):
    r = np.random.default_rng(seed)
    return r.uniform(0.5, 1.5, (H, 128)).astype(np.float32), r.uniform(0.5, 1.5, (H, 128)).astype(np.float32)


def run_case(sa, q, k, v, grid, bq, bk, keep, mode, layout="bhld", eps=1e-6, theta=10000.0, seed=0):
    """q, k, v: float32 numpy [B, H, L, d] (raw projections). Runs the fused call and checks it."""
    B, H, L, d = q.shape
    qb, kb, vb = bf16(q), bf16(k), bf16(v)
    if layout == "blhd":
        dev = [x.transpose(1, 2).contiguous().cuda().transpose(1, 2) for x in (qb, kb, vb)]
    else:
        dev = [x.cuda() for x in (qb, kb, vb)]
    gq, gk = gains(seed, H)
    pro = {"q_gain": torch.from_numpy(gq).cuda(), "k_gain": torch.from_numpy(gk).cuda(), "eps": eps,
           "grid": grid, "theta": theta}
    pbytes = sa.plan_prologue_workspace_bytes(B, H, L, d, bq, bk, grid)
    pws = torch.empty(pbytes, dtype=torch.uint8, device="cuda")
    plan, ws = sa.plan_prepare(*dev, bq, bk, keep, mode, plan_workspace=pws, prologue=pro)
    out = sa.attend(dev[0], plan, ws, bq, bk, mode)
    torch.cuda.synchronize()
    # oracle, from the bf16 inputs the GPU read
    qv, kv, vv = (x.float().numpy() for x in (qb, kb, vb))
    Qp = po.qk_prologue(qv, gq, eps, grid, theta)
    Kp = po.qk_prologue(kv, gk, eps, grid, theta)
    nQ, nK = sa.num_blocks(L, bq), sa.num_blocks(L, bk)
    qm, km = oracle.pool_block_means(Qp, bq), oracle.pool_block_means(Kp, bk)
    pw = pws.cpu().numpy()
    gqm = pw[:B * H * nQ * d * 8].view(np.float64).reshape(B, H, nQ, d)
    off = -(-B * H * nQ * d * 8 // 256) * 256
    gkm = pw[off:off + B * H * nK * d * 8].view(np.float64).reshape(B, H, nK, d)
    # fp64 sums of the same fp32 values in another order: |error| <= (n - 1) * 2^-53 * sum|x| / n
    for got, want, X, blk, name in ((gqm, qm, Qp, bq, "Q means"), (gkm, km, Kp, bk, "K means")):
        bound = (blk - 1) * 2.0 ** -53 * oracle.pool_block_means(np.abs(X), blk)
        err = np.abs(got - want)
        assert np.all(err <= bound), f"{name}: error {err.max():.2e} beyond the summation bound"
    nk = plan.shape[-1]
    mag = np.abs(qm) @ np.swapaxes(np.abs(km), -1, -2)
    excused = chk.compare_plan(plan.cpu().numpy(), oracle.block_scores(qm, km), nk, mag)
    lay = sa.forward_layout(B, H, L, d, bq, bk, mode)
    wsn = ws.cpu().numpy()
    quant = oracle.quantize_fp8_blocks if mode == "fp8" else oracle.quantize_int8_blocks
    Qh, sq = quant(Qp, bq)
    Kh, sk = quant(Kp, bk)
    Vq, sv = oracle.quantize_fp8_blocks(vv, bk)
    gqh, gq_pad = chk.decode_q_int8(wsn, lay, B, H, L, bq)
    gkh, gk_pad = chk.decode_k(wsn, lay, B, H, L, bk)
    gvh, _ = chk.decode_vt_fp8(wsn, lay, B, H, L, bk)
    gsq, gsk, gsv = chk.scales(wsn, lay, B, H)
    assert np.array_equal(gsq, sq) and np.array_equal(gsk, sk), "Q/K block scales"
    assert np.array_equal(gsv, sv), "V block scales"
    if mode == "fp8":
        assert np.array_equal(gqh.view(np.uint8), oracle.e4m3_bits(Qh)), "Q codes"
        assert np.array_equal(gkh, oracle.e4m3_bits(Kh)), "K codes"
    else:
        assert np.array_equal(gqh, Qh), "Q codes"
        assert np.array_equal(gkh.view(np.int8), Kh), "K codes"
    assert np.array_equal(gvh, oracle.e4m3_bits(Vq)), "V codes"
    assert not gq_pad.any() and not gk_pad.any()
    # the codes against those of the fp64 definitions of RMSNorm and 3-D RoPE (not the fp32
    # reading): equal except where the fp32 operations can cross a rounding boundary
    for name, gcodes, X, gain, blk in (("Q", gqh, qv, gq, bq), ("K", gkh, kv, gk, bk)):
        Y64, bnd = po.qk_prologue64(X, gain, eps, grid, theta)
        vals = (oracle.e4m3_decode(gcodes.view(np.uint8)) if mode == "fp8" else gcodes.view(np.int8))
        exc, tot = chk.codes_against_definition(vals, Y64, bnd, blk, mode, where=f"{name} ")
        say(f"  {name} codes vs the fp64 definitions: {exc} of {tot} differ, each at a rounding boundary")
        assert exc <= max(4, tot // 10000)
    # attention on the GPU's own plan, a few query blocks per head
    pn = plan.cpu().numpy()
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in sorted({0, nQ // 2, nQ - 1})]
    got = out.float().cpu().numpy()
    r = chk.check_quantized(got, Qh, sq, Kh, sk, Vq, sv, pn, bq, bk, rows=rows, qk_fp8=mode == "fp8")
    print("  " + chk.fmt(r), flush=True)
    return excused


CASES = [
    # name, B, H, grid, bq, bk, keep, mode, layout
    ("L1000_q128_k64", 1, 2, (10, 10, 10), 128, 64, 0.2, "int8fp8", "bhld"),
    ("L777_q64_k128", 1, 3, (7, 111, 1), 64, 128, 0.3, "int8fp8", "bhld"),
    ("L1500_q128_k128_B2", 2, 2, (6, 10, 25), 128, 128, 0.34, "int8fp8", "blhd"),
    ("L1024_fp8", 1, 2, (4, 16, 16), 64, 64, 0.25, "fp8", "bhld"),
    ("L50_single_block", 1, 2, (2, 5, 5), 128, 64, 0.5, "int8fp8", "bhld"),
    ("L960_1d_time", 1, 2, (960, 1, 1), 128, 64, 0.2, "fp8", "bhld"),
]


@pytest.mark.parametrize("name,B,H,grid,bq,bk,keep,mode,layout", CASES, ids=[c[0] for c in CASES])
def test_prologue_parity(sa, name, B, H, grid, bq, bk, keep, mode, layout):
    say(f"prologue {name}: B={B} H={H} grid={grid} bq={bq} bk={bk} keep={keep} {mode} {layout}")
    cfg = GridConfig(name, B, H, grid, 128, bq, bk, (keep,), (0.5,), "bf16", mode, 21)
    q, k, v = make_qkv(cfg)
    # raw projections: scaled per head so the norm has something to undo
    q *= np.arange(1, H + 1, dtype=np.float32)[None, :, None, None] * 3
    k *= 0.25
    excused = run_case(sa, q, k, v, grid, bq, bk, keep, mode, layout, seed=len(name))
    say(f"  plan rows excused by the near-tie band: {excused}")


def test_prologue_zero_rows_and_wide_eps(sa):
    cfg = GridConfig("zeros", 1, 2, (3, 7, 9), 128, 64, 64, (0.3,), (0.5,), "bf16", "int8fp8", 5)
    q, k, v = make_qkv(cfg)
    q[0, 0, 10:20] = 0.0  # zero rows normalize to zero
    k[0, 1, :64] = 0.0    # an all-zero K block: scale 0, codes 0
    run_case(sa, q, k, v, cfg.grid, 64, 64, 0.3, "int8fp8", eps=0.5, theta=500.0, seed=3)


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy()


BF16_CASES = [
    # name, B, H, grid, bq, bk, keep, layout
    ("L1000_q128_k64", 1, 2, (10, 10, 10), 128, 64, 0.2, "bhld"),
    ("L777_q64_k128", 1, 3, (7, 111, 1), 64, 128, 0.3, "blhd"),
    ("L50_single_block", 1, 2, (2, 5, 5), 128, 64, 0.5, "bhld"),
]


@pytest.mark.parametrize("name,B,H,grid,bq,bk,keep,layout", BF16_CASES, ids=[c[0] for c in BF16_CASES])
def test_prologue_bf16_mode(sa, name, B, H, grid, bq, bk, keep, layout):
    """bf16 mode: the same normalized, rotated fp32 values (block means and plan as in the
    quantized modes), rounded to bf16 (RNE) for the bf16 attention: the workspace's Q and K
    bit-exact against the oracle's values rounded to bf16, V untouched; within the rounding band
    of the fp64 definitions; attention within the bf16 bars of exact attention over those
    operands; a plain prepare on the same workspace switches the attention back to the caller's Q."""
    say(f"prologue bf16 {name}: B={B} H={H} grid={grid} bq={bq} bk={bk} keep={keep} {layout}")
    cfg = GridConfig(name, B, H, grid, 128, bq, bk, (keep,), (0.5,), "bf16", "bf16", 31)
    q, k, v = make_qkv(cfg)
    q *= np.arange(1, H + 1, dtype=np.float32)[None, :, None, None] * 3
    k *= 0.25
    L, d = q.shape[2], q.shape[3]
    qb, kb, vb = bf16(q), bf16(k), bf16(v)
    if layout == "blhd":
        dev = [x.transpose(1, 2).contiguous().cuda().transpose(1, 2) for x in (qb, kb, vb)]
    else:
        dev = [x.cuda() for x in (qb, kb, vb)]
    gq, gk = gains(len(name), H)
    eps, theta = 1e-6, 10000.0
    pro = {"q_gain": torch.from_numpy(gq).cuda(), "k_gain": torch.from_numpy(gk).cuda(), "eps": eps,
           "grid": grid, "theta": theta}
    pws = torch.empty(sa.plan_prologue_workspace_bytes(B, H, L, d, bq, bk, grid), dtype=torch.uint8, device="cuda")
    plan, ws = sa.plan_prepare(*dev, bq, bk, keep, "bf16", plan_workspace=pws, prologue=pro)
    out = sa.attend(dev[0], plan, ws, bq, bk, "bf16")
    torch.cuda.synchronize()
    qv, kv, vv = (x.float().numpy() for x in (qb, kb, vb))
    Qp = po.qk_prologue(qv, gq, eps, grid, theta)
    Kp = po.qk_prologue(kv, gk, eps, grid, theta)
    nQ, nK = sa.num_blocks(L, bq), sa.num_blocks(L, bk)
    qm, km = oracle.pool_block_means(Qp, bq), oracle.pool_block_means(Kp, bk)
    pw = pws.cpu().numpy()
    gqm = pw[:B * H * nQ * d * 8].view(np.float64).reshape(B, H, nQ, d)
    off = -(-B * H * nQ * d * 8 // 256) * 256
    gkm = pw[off:off + B * H * nK * d * 8].view(np.float64).reshape(B, H, nK, d)
    for got, want, X, blk, nm in ((gqm, qm, Qp, bq, "Q means"), (gkm, km, Kp, bk, "K means")):
        bound = (blk - 1) * 2.0 ** -53 * oracle.pool_block_means(np.abs(X), blk)
        assert np.all(np.abs(got - want) <= bound), nm
    nk = plan.shape[-1]
    mag = np.abs(qm) @ np.swapaxes(np.abs(km), -1, -2)
    excused = chk.compare_plan(plan.cpu().numpy(), oracle.block_scores(qm, km), nk, mag)
    lay = sa.forward_layout(B, H, L, d, bq, bk, "bf16")
    wsn = ws.cpu().numpy()
    assert wsn[lay["sq_off"]:lay["sq_off"] + 4].view(np.int32)[0] == 1, "Q-source word"
    nq_rows = nQ * bq
    gq16 = wsn[lay["q_off"]:lay["q_off"] + B * H * nq_rows * d * 2].view(np.int16).reshape(B, H, nq_rows, d)
    gk16, gk_pad = chk.decode_k(wsn, lay, B, H, L, bk, esize=2)
    gk16 = np.ascontiguousarray(gk16).view(np.int16)
    assert np.array_equal(gq16[:, :, :L], _bf16_bits(Qp)), "Q (bf16)"
    assert not gq16[:, :, L:].any() and not gk_pad.any(), "pad rows"
    assert np.array_equal(gk16, _bf16_bits(Kp)), "K (bf16)"
    gv, _ = chk.decode_vt_bf16(wsn, lay, B, H, L, bk)
    assert np.array_equal(np.ascontiguousarray(gv).view(np.int16), _bf16_bits(vv)), "V (bf16)"
    to_f = lambda bits: torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).float().numpy()
    for nm, gbits, X, gain, blk in (("Q", gq16[:, :, :L], qv, gq, bq), ("K", gk16, kv, gk, bk)):
        Y64, bnd = po.qk_prologue64(X, gain, eps, grid, theta)
        exc, tot = chk.codes_against_definition(to_f(gbits), Y64, bnd, blk, "bf16", where=f"{nm} ")
        say(f"  {nm} bf16 values vs the fp64 definitions: {exc} of {tot} differ, each at a rounding boundary")
        assert exc <= max(4, tot // 10000)
    pn = plan.cpu().numpy()
    want = oracle.attend_exact(to_f(_bf16_bits(Qp)), to_f(_bf16_bits(Kp)), vv, pn, bq, bk)
    got = out.float().cpu().numpy()
    err, mx = chk.rel_l2(got, want), np.abs(got - want).max()
    say(f"  plan rows excused {excused}; attention rel-L2 {err:.2e} max-abs {mx:.2e}")
    assert err <= 1e-2 and mx <= 2e-2
    # a plain prepare on the same workspace: the attention reads the caller's Q again
    sa.prepare(*dev, bq, bk, "bf16", workspace=ws)
    out2 = sa.attend(dev[0], plan, ws, bq, bk, "bf16")
    ref = sa.forward(*dev, plan, bq, bk, "bf16")
    torch.cuda.synchronize()
    assert torch.equal(out2, ref)


def test_720p_prologue_sampled(sa):
    """The 720p workload with the prologue in the benchmark's launch configuration; sampled heads
    and query blocks recomputed by the oracle from the same inputs."""
    cfg = CONFIGS["720p"]
    B, H, L, d, bq, bk = cfg.B, cfg.H, cfg.L, cfg.d, cfg.block_q, cfg.block_k
    say(f"720p prologue: B={B} H={H} L={L}")
    from tests.test_gpu_fullsize import upload
    qd, kd, vd = upload(cfg)
    gq, gk = gains(7, H)
    pro = {"q_gain": torch.from_numpy(gq).cuda(), "k_gain": torch.from_numpy(gk).cuda(), "eps": 1e-6,
           "grid": cfg.grid}
    plan, ws = sa.plan_prepare(qd, kd, vd, bq, bk, cfg.keep, "int8fp8", prologue=pro)
    out = sa.attend(qd, plan, ws, bq, bk, "int8fp8")
    torch.cuda.synchronize()
    lay = sa.forward_layout(B, H, L, d, bq, bk, "int8fp8")
    nk = plan.shape[-1]
    for h, i in ((0, 0), (17, 300), (39, 590)):
        sl = lambda x: x[0:1, h:h + 1].float().cpu().numpy()
        Qp = po.qk_prologue(sl(qd), gq[h:h + 1], 1e-6, cfg.grid)
        Kp = po.qk_prologue(sl(kd), gk[h:h + 1], 1e-6, cfg.grid)
        S, mag = chk.pooled_scores(Qp, Kp, bq, bk)
        ph = plan[0:1, h:h + 1].cpu().numpy()
        excused = chk.compare_plan(ph, S, nk, mag, label=f"head {h} ")
        Qh, sq = oracle.quantize_int8_blocks(Qp, bq)
        Kh, sk = oracle.quantize_int8_blocks(Kp, bk)
        Vq, sv = oracle.quantize_fp8_blocks(sl(vd), bk)
        # the head's quantized Q block i and its scales, straight from the workspace
        nQ, nK = lay["nQ"], lay["nK"]
        wq = ws[lay["q_off"] + ((h * nQ + i) * bq) * d: lay["q_off"] + ((h * nQ + i + 1) * bq) * d]
        r1 = min(bq, L - i * bq)
        got_q = wq.cpu().numpy().view(np.int8).reshape(bq, d)[:r1]
        assert np.array_equal(got_q, Qh[0, 0, i * bq:i * bq + r1]), (h, i)
        wsk = ws[lay["sk_off"] + 4 * h * nK: lay["sk_off"] + 4 * (h + 1) * nK].cpu().numpy().view(np.float32)
        assert np.array_equal(wsk, sk[0, 0]), h
        r0 = i * bq
        got = np.full(Qh.shape, np.nan)
        got[0, 0, r0:r0 + r1] = out[0, h, r0:r0 + r1].float().cpu().numpy()
        r = chk.check_quantized(got, Qh, sq, Kh, sk, Vq, sv, ph, bq, bk, rows=[(0, 0, i)])
        say(f"  head {h} block {i}: plan rows excused {excused}; " + chk.fmt(r))
        assert excused <= 5
