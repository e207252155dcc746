"""Parity at the full sizes of the long-sequence and keep-sweep workloads, on sampled outputs.

The whole path runs on the GPU at the workload's size, in the launch configuration the
benchmark times (one plan launch sequence, then prepare and attend, each covering every
batch item and head); the oracle then recomputes sampled plan rows and query blocks one by
one from the same device inputs copied back to the host.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, head_qkv
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


def upload(cfg):
    """The workload's seeded inputs as bf16 [B, H, L, d] device tensors, drawn head by head."""
    dev = torch.device("cuda:0")
    qkv = [torch.empty((cfg.B, cfg.H, cfg.L, cfg.d), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    for b in range(cfg.B):
        sigma = cfg.sigmas[b % len(cfg.sigmas)]
        for h in range(cfg.H):
            for t, x in zip(qkv, head_qkv(cfg.seed, b, h, cfg.grid, cfg.d, sigma)):
                t[b, h].copy_(torch.from_numpy(np.ascontiguousarray(x)))
    torch.cuda.synchronize()
    return qkv


def run_and_check(sa, cfg, keep, qkv, samples, mode="int8fp8"):
    qd, kd, vd = qkv
    bq, bk = cfg.block_q, cfg.block_k
    nQ, nK = sa.num_blocks(cfg.L, bq), sa.num_blocks(cfg.L, bk)
    nk = oracle.n_keep(nK, keep)
    say(f"{cfg.name} keep={keep} {mode}: plan + prepare + attend, B={cfg.B} H={cfg.H} L={cfg.L} n_keep={nk}")
    p = sa.plan(qd, kd, bq, bk, keep)
    ws = sa.prepare(qd, kd, vd, bq, bk, mode)
    out = sa.attend(qd, p, ws, bq, bk, mode)
    torch.cuda.synchronize()
    pn = p.cpu().numpy()
    assert pn.shape == (cfg.B, cfg.H, nQ, nk)
    assert torch.isfinite(out.float()).all()
    del ws
    for b, h, i in samples:
        sl = lambda x: x[b:b + 1, h:h + 1].float().cpu().numpy()
        qv, kv, vv = sl(qd), sl(kd), sl(vd)
        ph = pn[b:b + 1, h:h + 1]
        S, mag = chk.pooled_scores(qv, kv, bq, bk)
        excused = chk.compare_plan(ph, S, nk, mag, label=f"b={b} h={h} ")
        qk_quant = oracle.quantize_fp8_blocks if mode == "fp8" else oracle.quantize_int8_blocks
        Qh, sq = qk_quant(qv, bq)
        Kh, sk = qk_quant(kv, bk)
        Vq, sv = oracle.quantize_fp8_blocks(vv, bk)
        r0, r1 = bq * i, min(bq * i + bq, cfg.L)
        got = np.full(Qh.shape, np.nan)
        got[0, 0, r0:r1] = out[b, h, r0:r1].float().cpu().numpy()
        r = chk.check_quantized(got, Qh, sq, Kh, sk, Vq, sv, ph, bq, bk, rows=[(0, 0, i)],
                                qk_fp8=mode == "fp8")
        say(f"  b={b} h={h} block {i}: plan rows excused {excused}; " + chk.fmt(r))
        assert excused <= 5


def test_long_sequence_sampled(sa):
    cfg = CONFIGS["long"]
    say(f"generating {cfg.name} inputs (B={cfg.B} H={cfg.H} L={cfg.L})")
    qkv = upload(cfg)
    run_and_check(sa, cfg, 0.1, qkv, [(0, 0, 0), (0, 21, 480), (0, 39, 959)])
    run_and_check(sa, cfg, 1.0, qkv, [(0, 3, 10), (0, 30, 959)])  # every block kept: dense


def test_keep_sweep_sampled(sa):
    cfg = CONFIGS["sweep"]
    say(f"generating {cfg.name} inputs (B={cfg.B} H={cfg.H} L={cfg.L}, sigma {cfg.sigmas})")
    qkv = upload(cfg)
    samples = {0.05: [(0, 2, 590), (1, 37, 7)], 0.1: [(0, 11, 300), (1, 0, 590)],
               0.2: [(0, 39, 44), (1, 19, 222)], 0.5: [(0, 8, 590), (1, 26, 400)],
               1.0: [(0, 31, 150), (1, 5, 590)]}
    assert tuple(samples) == tuple(cfg.keeps)
    for keep in cfg.keeps:
        run_and_check(sa, cfg, keep, qkv, samples[keep])


def test_720p_all_fp8_mode_sampled(sa):
    cfg = CONFIGS["720p"]
    say(f"generating {cfg.name} inputs (B={cfg.B} H={cfg.H} L={cfg.L})")
    qkv = upload(cfg)
    run_and_check(sa, cfg, cfg.keep, qkv, [(0, 0, 0), (0, 19, 333), (0, 39, 590)], mode="fp8")
