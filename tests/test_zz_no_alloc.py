"""The plan entry point that allocates nothing (sparse_attn_plan_noalloc), through the C ABI:
its plans equal those of sparse_attn_plan (bit for bit: integer block indices) on consecutive
calls that share the library's fixed scratch, the second call on a smaller input."""
import sys

import numpy as np
import pytest
import torch

from synth import CONFIGS, GridConfig, head_qkv, make_qkv

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


def _inputs_720p_share(heads=5):
    """The 720p workload's first `heads` heads (one GPU's share of 40 heads over 8 GPUs)."""
    cfg = CONFIGS["720p"]
    q = torch.empty((1, heads, cfg.L, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)
    for h in range(heads):
        hq, hk, _ = head_qkv(cfg.seed, 0, h, cfg.grid, cfg.d, cfg.sigmas[0])
        q[0, h].copy_(torch.from_numpy(np.ascontiguousarray(hq)))
        k[0, h].copy_(torch.from_numpy(np.ascontiguousarray(hk)))
    return q, k, cfg.block_q, cfg.block_k, cfg.keep


def _inputs_small():
    cfg = GridConfig("L1000_q128_k64", 1, 2, (10, 10, 10), 128, 128, 64, (0.2,), (0.5,), "bf16", "int8fp8", 11)
    q, k, _ = make_qkv(cfg)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)
    return dev(q), dev(k), cfg.block_q, cfg.block_k, cfg.keep


def _check(sa, q, k, bq, bk, keep, name):
    B, H, L, _ = q.shape
    nQ, nK = sa.num_blocks(L, bq), sa.num_blocks(L, bk)
    nk = sa.n_keep(nK, keep)
    assert sa.plan_workspace_bytes(B, H, L, 128, bq, bk) <= sa.plan_noalloc_max_bytes()
    out = torch.full((B, H, nQ, nk), -7, dtype=torch.int32, device="cuda")  # every entry must be written
    sa.plan_noalloc(q, k, bq, bk, keep, out)
    want = sa.plan(q, k, bq, bk, keep)
    torch.cuda.synchronize()
    assert torch.equal(out, want), name
    say(f"  {name}: plan [{B}, {H}, {nQ}, {nk}] equals sparse_attn_plan's")


def test_noalloc_plan_equals_plan_on_consecutive_calls(sa):
    say("no-alloc plan: 720p shape, 5 heads, then a 2-head L=1000 input, then the 5 heads again")
    big = _inputs_720p_share()
    small = _inputs_small()
    _check(sa, *big, "720p 5 heads")
    _check(sa, *small, "L1000 2 heads (smaller, second call)")
    _check(sa, *big, "720p 5 heads (after the smaller call)")


def test_noalloc_plan_refuses_shapes_beyond_its_scratch(sa):
    cfg = CONFIGS["480p"]
    q = torch.zeros((1, 40, cfg.L, 128), dtype=torch.bfloat16, device="cuda")
    nk = sa.n_keep(sa.num_blocks(cfg.L, 64), cfg.keep)
    out = torch.empty((1, 40, sa.num_blocks(cfg.L, 128), nk), dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError, match="noalloc"):
        sa.plan_noalloc(q, q, 128, 64, cfg.keep, out)
