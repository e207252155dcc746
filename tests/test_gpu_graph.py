"""The library's calls under HIP graph capture.

The library allocates, copies, clears and synchronises nothing: every call is argument checks
on the host and kernel launches on the caller's stream, so a graph can hold it. Each test
captures a sequence of calls once, then replays the graph several times on new inputs written
into the captured buffers, with eager work and synchronisations between the replays, and checks
every replay bit for bit against the same calls made eagerly on separate buffers. (Parity with
the oracle is the other test files' job; this checks that capture changes nothing.)
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from synth import GridConfig, make_qkv

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


def capture(fn):
    """Warm fn up on a side stream (torch's capture protocol), then capture one call of it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def same_bits(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("mode", ["int8fp8", "fp8", "bf16"])
def test_step_replays_equal_eager(sa, mode):
    """plan_prepare + attend captured once, replayed on three new inputs."""
    cfg = GridConfig("graph_L1000", 1, 2, (10, 10, 10), 128, 128, 64, (0.2,), (0.5,), "bf16", mode, 1)
    B, H, L, bq, bk, keep = cfg.B, cfg.H, cfg.L, cfg.block_q, cfg.block_k, 0.2
    say(f"graph step {mode}: B={B} H={H} L={L} bq={bq} bk={bk} keep={keep}")
    nQ, nK = sa.num_blocks(L, bq), sa.num_blocks(L, bk)
    nk = sa.n_keep(nK, keep)

    def buffers():
        return (torch.empty((B, H, nQ, nk), dtype=torch.int32, device="cuda"),
                torch.empty(sa.plan_workspace_bytes(B, H, L, 128, bq, bk), dtype=torch.uint8, device="cuda"),
                torch.empty(sa.forward_workspace_bytes(B, H, L, 128, bq, bk, mode), dtype=torch.uint8,
                            device="cuda"),
                torch.empty((B, H, L, 128), dtype=torch.bfloat16, device="cuda"))

    q, k, v = (torch.empty((B, H, L, 128), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    cap, ref = buffers(), buffers()

    def step(bufs):
        plan, wsp, wsf, out = bufs
        sa.plan_prepare(q, k, v, bq, bk, keep, mode, out=plan, plan_workspace=wsp, workspace=wsf)
        sa.attend(q, plan, wsf, bq, bk, mode, out=out)

    def fill(seed):
        for t, x in zip((q, k, v), make_qkv(dataclasses.replace(cfg, seed=seed))):
            t.copy_(torch.from_numpy(x).to(torch.bfloat16))

    fill(100)
    g = capture(lambda: step(cap))
    for seed in (101, 102, 103):
        fill(seed)
        step(ref)  # eager, on separate buffers
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"  replay on inputs {seed}: plan equal {torch.equal(cap[0], ref[0])}, "
            f"output equal {same_bits(cap[3], ref[3])}")
        assert torch.equal(cap[0], ref[0])
        assert same_bits(cap[3], ref[3])
        assert torch.isfinite(cap[3].float()).all()


def test_nvfp4_quantize_and_gemm_replay_equal_eager(sa):
    """The activation quantizer and the NVFP4 GEMM (with bias) captured once, replayed three times."""
    M, N, K = 300, 264, 512
    say(f"graph NVFP4: M={M} N={N} K={K}")
    rng = np.random.default_rng(7)
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    w = torch.from_numpy(rng.standard_normal((N, K)).astype(np.float32)).to("cuda").to(torch.bfloat16)
    bias = torch.from_numpy(rng.standard_normal(N).astype(np.float32)).to("cuda").to(torch.bfloat16)
    wq = sa.nvfp4_quantize(w)

    def buffers():
        return ((torch.empty((M, K // 2), dtype=torch.uint8, device="cuda"),
                 torch.empty((M, K // 16), dtype=torch.uint8, device="cuda"),
                 torch.empty(1, dtype=torch.float32, device="cuda")),
                torch.empty(4096, dtype=torch.uint8, device="cuda"),
                torch.empty((M, N), dtype=torch.bfloat16, device="cuda"))

    cap, ref = buffers(), buffers()

    def run(bufs):
        a, ws, y = bufs
        sa.nvfp4_quantize(x, out=a, workspace=ws)
        sa.nvfp4_gemm(a, wq, bias, out=y)

    x.copy_(torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16))
    g = capture(lambda: run(cap))
    for r in range(3):
        x.copy_(torch.from_numpy((rng.standard_normal((M, K)) * 10.0 ** (r - 1)).astype(np.float32))
                .to(torch.bfloat16))
        run(ref)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eq = [same_bits(c, e) for c, e in zip(cap[0] + (cap[2],), ref[0] + (ref[2],))]
        say(f"  replay {r}: codes, scales, tensor scale, output equal {eq}")
        assert all(eq)
