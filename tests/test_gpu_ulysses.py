"""Light-Ulysses FP8 exchange payload: the pack and unpack kernels against the oracle, with P
peers emulated on one GPU (each peer's tensors are views of one full tensor; the all-to-all is
replaced by copying chunk r of every sender into the receive buffer of peer r).

Bars: payload codes and scale bytes bit-exact; unpacked tensors bit-exact against the oracle's
dequantized rows rounded to bf16; the sequence-parallel attention step (exchange, attention
on each peer's heads, exchange back) bit-exact against one attention over all heads of the
same dequantized inputs, exchanged back by the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from tests import sa_checks as chk
from oracle import ulysses as uo
from synth import GridConfig, make_qkv, wide_rows

pytestmark = pytest.mark.gpu
D = 128


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


def device_bf16(x, layout="bhld"):
    """bf16 device tensor of logical shape [B, H, L, D] (RNE cast), stored [B,H,L,D] or [B,L,H,D]."""
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)
    if layout == "blhd":
        return t.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    return t.cuda()


def host(t):
    return t.float().cpu().numpy()


def split_payload(pay, chunk, P, B, lmax, hc, T):
    """(codes as E4M3 values [P][B][Lmax][hc][T][D], exponents [P][B][Lmax][hc][T]) of a payload."""
    raw = pay.cpu().numpy()
    rows = B * lmax * hc * T
    codes = np.empty((P, B, lmax, hc, T, D), np.float32)
    exps = np.empty((P, B, lmax, hc, T), np.int32)
    for c in range(P):
        base = c * chunk
        cb = torch.from_numpy(raw[base:base + rows * D].copy()).view(torch.float8_e4m3fn).float().numpy()
        codes[c] = cb.reshape(B, lmax, hc, T, D)
        exps[c] = raw[base + rows * D:base + rows * (D + 1)].astype(np.int32).reshape(B, lmax, hc, T) - 127
    return codes, exps


def exchange(sends, chunk):
    """All-to-all with equal splits, on one GPU: peer r receives chunk r of every sender, in order."""
    P = len(sends)
    return [torch.cat([s[r * chunk:(r + 1) * chunk] for s in sends]) for r in range(P)]


def assert_same(got, want, what):
    bad = ~((got == want) | (np.isnan(got) & np.isnan(want)))
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} differ, first at {np.argwhere(bad)[0]}"


def seq_to_head_round(sa, full_dev, full_host, L, P, h0, hc):
    """Pack every peer's shard, check each payload against the oracle, exchange, unpack; returns
    the head-side tensors of every peer [B, hc, L, D] (device)."""
    B, H = full_dev[0].shape[:2]
    T = len(full_dev)
    bounds, lmax = uo.shard_bounds(L, P)
    chunk, total = sa.ulysses_payload_bytes(B, hc, L, P, T)
    sends = []
    for r, (lo, hi) in enumerate(bounds):
        pay = sa.ulysses_pack_seq([x[:, :, lo:hi] for x in full_dev], L, P, r, h0, hc)
        assert pay.numel() == total
        codes, exps = split_payload(pay, chunk, P, B, lmax, hc, T)
        want_c, want_e = uo.payload([x[:, :, lo:hi] for x in full_host], L, r, P, h0, hc)
        assert_same(codes, want_c, f"codes of peer {r}")
        assert_same(exps, want_e, f"scale bytes of peer {r}")
        sends.append(pay)
    outs = []
    for r, recv in enumerate(exchange(sends, chunk)):
        y = [torch.full((B, hc, L, D), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(T)]
        sa.ulysses_unpack_head(recv, P, y)
        outs.append(y)
    torch.cuda.synchronize()
    return outs


SEQ_CASES = [
    # B, H, L, P, T, layout, head chunks (h0, hc); None = all heads of a group at once
    (2, 8, 1000, 4, 3, "bhld", None),       # even shards of 250 tokens
    (1, 6, 103, 3, 2, "bhld", [(0, 1), (1, 1)]),  # ragged: shards of 35, 35, 33; one head a chunk
    (1, 4, 77, 1, 1, "bhld", None),         # one peer: the payload is every row of the tensor
    (1, 16, 1031, 8, 3, "blhd", [(0, 1), (1, 1)]),  # [B, L, H, D] storage, 129-token shards
]


@pytest.mark.parametrize("B,H,L,P,T,layout,chunks", SEQ_CASES)
def test_sequence_to_head_exchange(sa, B, H, L, P, T, layout, chunks):
    say(f"seq->head B={B} H={H} L={L} P={P} T={T} {layout} chunks={chunks}")
    full_host = [host(device_bf16(wide_rows(100 + i, (B, H, L, D)))) for i in range(T)]
    full_dev = [device_bf16(x, layout) for x in full_host]
    hp = H // P
    want = uo.seq_to_head(full_host, P)  # per peer, per tensor: [B, hp, L, D] dequantized
    for h0, hc in chunks or [(0, hp)]:
        got = seq_to_head_round(sa, full_dev, full_host, L, P, h0, hc)
        for r in range(P):
            for ti in range(T):
                assert_same(host(got[r][ti]), oracle.bf16_rne(want[r][ti][:, h0:h0 + hc]).astype(np.float32),
                            f"peer {r} tensor {ti} heads [{h0}, {h0 + hc})")


HEAD_CASES = [
    (1, 8, 1000, 4, 1, None),
    (2, 6, 103, 3, 1, [(0, 1), (1, 1)]),
    (1, 16, 1031, 8, 2, None),
]


@pytest.mark.parametrize("B,H,L,P,T,chunks", HEAD_CASES)
def test_head_to_sequence_exchange(sa, B, H, L, P, T, chunks):
    say(f"head->seq B={B} H={H} L={L} P={P} T={T} chunks={chunks}")
    hp = H // P
    bounds, lmax = uo.shard_bounds(L, P)
    per_peer_host = [[host(device_bf16(wide_rows(200 + 10 * r + ti, (B, hp, L, D)))) for ti in range(T)]
                     for r in range(P)]
    per_peer_dev = [[device_bf16(x) for x in xs] for xs in per_peer_host]
    shards = [[torch.full((B, H, hi - lo, D), float("nan"), dtype=torch.bfloat16, device="cuda")
               for _ in range(T)] for lo, hi in bounds]
    for h0, hc in chunks or [(0, hp)]:
        chunk, _ = sa.ulysses_payload_bytes(B, hc, L, P, T)
        sends = []
        for r in range(P):
            pay = sa.ulysses_pack_head([x[:, h0:h0 + hc] for x in per_peer_dev[r]], P)
            codes, exps = split_payload(pay, chunk, P, B, lmax, hc, T)
            want_c, want_e = uo.payload_back([x[:, h0:h0 + hc] for x in per_peer_host[r]], P)
            assert_same(codes, want_c, f"codes of peer {r}")
            assert_same(exps, want_e, f"scale bytes of peer {r}")
            sends.append(pay)
        for r, recv in enumerate(exchange(sends, chunk)):
            sa.ulysses_unpack_seq(recv, L, P, r, shards[r], h0, hc)
    torch.cuda.synchronize()
    for ti in range(T):
        want = uo.head_to_seq([per_peer_host[r][ti] for r in range(P)], L, P)
        for r in range(P):
            assert_same(host(shards[r][ti]), oracle.bf16_rne(want[r]).astype(np.float32), f"shard {r} tensor {ti}")


def test_unpack_seq_leaves_other_heads_alone(sa):
    B, H, L, P = 1, 8, 64, 2
    hp = H // P
    x = [device_bf16(wide_rows(300 + r, (B, hp, L, D))) for r in range(P)]
    chunk, _ = sa.ulysses_payload_bytes(B, 1, L, P, 1)
    sends = [sa.ulysses_pack_head([t[:, 2:3]], P) for t in x]
    shard = torch.full((B, H, L // P, D), 7.0, dtype=torch.bfloat16, device="cuda")
    sa.ulysses_unpack_seq(exchange(sends, chunk)[1], L, P, 1, [shard], 2, 1)
    torch.cuda.synchronize()
    got = host(shard)
    written = [c * hp + 2 for c in range(P)]
    for h in range(H):
        if h not in written:
            assert np.all(got[0, h] == 7.0), h
        else:
            assert not np.any(np.isnan(got[0, h]))


def test_sequence_parallel_attention_step(sa):
    """Tokens split over 4 peers: exchange to heads, attention on each peer's 2 heads, exchange
    back; equals attention over all 8 heads of the same dequantized inputs, exchanged back."""
    cfg = GridConfig("sp", 1, 8, (4, 16, 32), 128, 128, 64, (0.25,), (0.5,), "bf16", "int8fp8", 7)
    B, H, L, P = cfg.B, cfg.H, cfg.L, 4
    hp = H // P
    bounds, _ = uo.shard_bounds(L, P)
    full_host = [host(device_bf16(x)) for x in make_qkv(cfg)]
    full_dev = [device_bf16(x) for x in full_host]
    say(f"sequence-parallel step B={B} H={H} L={L} P={P}")
    heads = seq_to_head_round(sa, full_dev, full_host, L, P, 0, hp)  # checked against the oracle inside
    outs = []
    for r in range(P):
        q, k, v = heads[r]
        plan, ws = sa.plan_prepare(q, k, v, cfg.block_q, cfg.block_k, cfg.keep, "int8fp8")
        outs.append(sa.attend(q, plan, ws, cfg.block_q, cfg.block_k, "int8fp8"))
    # the same attention over all heads at once (heads never interact)
    qa, ka, va = [torch.cat([heads[r][ti] for r in range(P)], dim=1) for ti in range(3)]
    plan, ws = sa.plan_prepare(qa, ka, va, cfg.block_q, cfg.block_k, cfg.keep, "int8fp8")
    whole = sa.attend(qa, plan, ws, cfg.block_q, cfg.block_k, "int8fp8")
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=1), whole)
    chunk, _ = sa.ulysses_payload_bytes(B, hp, L, P, 1)
    sends = [sa.ulysses_pack_head([o], P) for o in outs]
    shards = [torch.empty((B, H, hi - lo, D), dtype=torch.bfloat16, device="cuda") for lo, hi in bounds]
    for r, recv in enumerate(exchange(sends, chunk)):
        sa.ulysses_unpack_seq(recv, L, P, r, [shards[r]])
    torch.cuda.synchronize()
    want = uo.head_to_seq([host(o) for o in outs], L, P)
    for r in range(P):
        assert_same(host(shards[r]), oracle.bf16_rne(want[r]).astype(np.float32), f"output shard {r}")
    # and the output is attention: compare one query block of one head with the quantized oracle
    b, h, i = 0, 5, 3
    qv, kv, vv = [host(t[b:b + 1, h:h + 1]) for t in (qa, ka, va)]
    Qh, sq = oracle.quantize_int8_blocks(qv, cfg.block_q)
    Kh, sk = oracle.quantize_int8_blocks(kv, cfg.block_k)
    Vq, sv = oracle.quantize_fp8_blocks(vv, cfg.block_k)
    ph = plan[b:b + 1, h:h + 1].cpu().numpy()
    r0, r1 = i * cfg.block_q, (i + 1) * cfg.block_q
    got = np.full(Qh.shape, np.nan)
    got[0, 0, r0:r1] = host(whole[b, h, r0:r1])
    chk.check_quantized(got, Qh, sq, Kh, sk, Vq, sv, ph, cfg.block_q, cfg.block_k, rows=[(0, 0, i)])


def test_720p_over_8_peers_sampled(sa):
    """The 720p shape (H=40, L=75600) over 8 peers at full size, Q, K, V in one payload: every
    peer packs its 9450-token shard, the exchange runs, every peer unpacks its 5 heads; sampled
    rows of every payload and every unpacked tensor checked against the oracle."""
    B, H, L, P = 1, 40, 75600, 8
    hp = H // P
    bounds, lmax = uo.shard_bounds(L, P)
    g = torch.Generator(device="cuda").manual_seed(5)
    full = [(torch.randn((B, H, L, D), generator=g, device="cuda") * s).to(torch.bfloat16) for s in (1.0, 3.0, 0.5)]
    say(f"720p over {P} peers: B={B} H={H} L={L}")
    chunk, _ = sa.ulysses_payload_bytes(B, hp, L, P, 3)
    sends = [sa.ulysses_pack_seq([x[:, :, lo:hi] for x in full], L, P, r) for r, (lo, hi) in enumerate(bounds)]
    recvs = exchange(sends, chunk)
    heads = []
    for r in range(P):
        y = [torch.empty((B, hp, L, D), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
        sa.ulysses_unpack_head(recvs[r], P, y)
        heads.append(y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = B * lmax * hp * 3
    for _ in range(64):
        r, c, t, hl, ti = (int(rng.integers(P)), int(rng.integers(P)), int(rng.integers(lmax)),
                           int(rng.integers(hp)), int(rng.integers(3)))
        lo, _ = bounds[r]
        src = host(full[ti][0, c * hp + hl, lo + t])
        q, e = uo.fp8_rows(src[None])
        i = (t * hp + hl) * 3 + ti
        raw = sends[r][c * chunk + i * D:c * chunk + (i + 1) * D].cpu()
        assert np.array_equal(raw.view(torch.float8_e4m3fn).float().numpy(), q[0])
        assert int(sends[r][c * chunk + rows * D + i]) == 127 + int(e[0])
        got = host(heads[c][ti][0, hl, lo + t])
        assert np.array_equal(got, oracle.bf16_rne(uo.dequant_rows(src[None])[0]).astype(np.float32))
