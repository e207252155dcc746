"""Oracle of the Light-Ulysses FP8 packing (test infrastructure: imported only by the tests,
the smoke run and the benchmark's CPU baseline).

Page "600倍加速，720p视频实时生成！单卡也能带的动14B模型", multi-card path, Light-Ulysses
paragraph: the token sequence is split over the GPUs; an all-to-all moves Q, K, V from the
sequence split to a head split before attention and the output back after it; the data sent
is FP8 both ways, and Q, K and V travel as one payload. Readings (the pages give no format):

* P peers; tokens in P contiguous shards of Lmax = ceil(L / P) (the last one shorter), heads
  in P contiguous groups of H / P (H divisible by P).
* Every row of d values (one token, one head, one tensor) is sent as E4M3 codes with one
  power-of-two scale 2^e, e = fp8_block_exponent(max |row|) (the same rule as the V blocks);
  the scale travels as its E8M0 byte 127 + e. The receiver rebuilds code * 2^e exactly.
* The payload a peer sends is [P destinations][B][Lmax][hc][T][d] codes and
  [P][B][Lmax][hc][T] scale bytes (T = 3 for Q, K, V; T = 1 for the output), rows past the
  end of a short shard zero, so every destination gets the same number of bytes.
* Head-by-head pipelining: a chunk of hc heads out of each group of H/P is one exchange
  (hc = H/P moves every head at once).

Parity unpinned against the pages (they print no payload); pinned to the definitions by the
tests in tests/test_oracle_pins.py.
"""
import numpy as np

from .blocksparse import e4m3_rne, fp8_block_exponent


def fp8_rows(x):
    """E4M3 grid values and exponents of every row (last axis) of x: (codes as values, e)."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).max(axis=-1)
    e = fp8_block_exponent(a).astype(np.int32)
    inv = np.exp2(-e.astype(np.float64)).astype(np.float32)
    q = e4m3_rne(np.clip((x * inv[..., None]).astype(np.float32), -448.0, 448.0))
    return q, e


def dequant_rows(x):
    """What a receiver rebuilds from a row sent in FP8: code * 2^e (exact)."""
    q, e = fp8_rows(x)
    return q.astype(np.float64) * np.exp2(e.astype(np.float64))[..., None]


def shard_bounds(L: int, peers: int):
    lmax = -(-L // peers)
    return [(r * lmax, min((r + 1) * lmax, L)) for r in range(peers)], lmax


def seq_to_head(tensors, peers: int):
    """What each peer holds after the sequence-to-head exchange of the given full tensors
    (each [B, H, L, d]): a list over peers of lists over tensors of [B, H/P, L, d] arrays."""
    B, H, L, d = tensors[0].shape
    assert H % peers == 0
    hp = H // peers
    deq = [dequant_rows(t) for t in tensors]
    return [[x[:, p * hp:(p + 1) * hp] for x in deq] for p in range(peers)]


def head_to_seq(per_peer, L: int, peers: int):
    """Inverse exchange of per-peer outputs (list over peers of [B, H/P, L, d]): what each peer
    holds afterwards, [B, H, L_r, d] for its token shard r."""
    bounds, _ = shard_bounds(L, peers)
    deq = [dequant_rows(x) for x in per_peer]
    full = np.concatenate(deq, axis=1)  # [B, H, L, d]
    return [full[:, :, lo:hi] for lo, hi in bounds]


def payload(tensors_local, L: int, rank: int, peers: int, head_begin: int = 0, head_count=None):
    """Payload a peer sends in the sequence-to-head exchange: its shard of each tensor
    ([B, H, L_r, d], the same order as in the payload) as (codes [P][B][Lmax][hc][T][d] values,
    exponents [P][B][Lmax][hc][T]). Destination p gets heads p*(H/P) + [head_begin,
    head_begin + hc) of every token of the shard (hc = head_count, all H/P heads by default: the
    head-by-head pipelining reading moves a head chunk per exchange)."""
    T = len(tensors_local)
    B, H, Lr, d = tensors_local[0].shape
    hp = H // peers
    hc = hp - head_begin if head_count is None else head_count
    bounds, lmax = shard_bounds(L, peers)
    assert Lr == bounds[rank][1] - bounds[rank][0]
    codes = np.zeros((peers, B, lmax, hc, T, d), np.float32)
    exps = np.zeros((peers, B, lmax, hc, T), np.int32)
    for ti, x in enumerate(tensors_local):
        q, e = fp8_rows(x)  # [B, H, Lr, d], [B, H, Lr]
        for p in range(peers):
            h0 = p * hp + head_begin
            codes[p, :, :Lr, :, ti] = np.transpose(q[:, h0:h0 + hc], (0, 2, 1, 3))
            exps[p, :, :Lr, :, ti] = np.transpose(e[:, h0:h0 + hc], (0, 2, 1))
    return codes, exps


def payload_back(tensors_heads, peers: int):
    """Payload a peer sends in the head-to-sequence exchange: its head chunk of each tensor
    ([B, hc, L, d], whole sequence) as (codes [P][B][Lmax][hc][T][d] values, exponents
    [P][B][Lmax][hc][T]); destination p gets the tokens of shard p."""
    T = len(tensors_heads)
    B, hc, L, d = tensors_heads[0].shape
    bounds, lmax = shard_bounds(L, peers)
    codes = np.zeros((peers, B, lmax, hc, T, d), np.float32)
    exps = np.zeros((peers, B, lmax, hc, T), np.int32)
    for ti, x in enumerate(tensors_heads):
        q, e = fp8_rows(x)  # [B, hc, L, d], [B, hc, L]
        for p, (lo, hi) in enumerate(bounds):
            codes[p, :, :hi - lo, :, ti] = np.transpose(q[:, :, lo:hi], (0, 2, 1, 3))
            exps[p, :, :hi - lo, :, ti] = np.transpose(e[:, :, lo:hi], (0, 2, 1))
    return codes, exps
