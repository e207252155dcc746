"""Plain numpy definition of block-mean-selected block-sparse attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by the tests,
the smoke check and the benchmark's CPU baseline, never by the library.

Arrays are numpy, logical layout [B, H, L, d]. Floating point is float64
unless a step says otherwise; the quantized simulation keeps every value that
decides an INT8 or FP8 code in float32, the precision the GPU decides it in.

Page short names used below:
  NEWS  = "600倍加速，720p视频实时生成！单卡也能带的动14B模型" (66bd.net article)
  GUIDE = "Run Wan2.2-A14B on One RTX 5090: 720p Video in 3.8s" (aoyii.com, English)
  WIKI  = "600 倍加速 720p 视频实时生成 — 单卡 14B 模型推理优化" (ai-engineering wiki)
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = 1.4426950408889634  # log2(e) to double precision
E4M3_MAX = 448.0  # largest finite OCP E4M3FN value (1.75 * 2^8)
TILE_KEYS = 64  # keys per online-softmax step of the quantized attention


# --------------------------------------------------------------------------
# Blocks of consecutive tokens
# --------------------------------------------------------------------------
def block_bounds(L: int, b: int):
    """[start, end) of every block of b consecutive tokens; the last may be short.

    Reading: the pages speak of blocks and tiles of the token sequence without a
    shape (NEWS, dynamic sparse quantized attention paragraph); a block here is a
    run of b consecutive tokens of the row-major flattened (t, y, x) grid, and a
    sequence length that is not a multiple of b leaves a shorter last block.
    """
    if L < 1 or b < 1:
        raise ValueError("L and b must be positive")
    n = -(-L // b)
    return [(i * b, min((i + 1) * b, L)) for i in range(n)]


# --------------------------------------------------------------------------
# O1  block means
# --------------------------------------------------------------------------
def pool_block_means(X, b: int):
    """Mean of X over each block of b tokens, per (batch, head): [B, H, n, d] float64.

    Follows NEWS (dynamic sparse quantized attention paragraph) and GUIDE
    (section 3): importance is estimated from block-level means of Q and K.
    The mean of a short last block divides by its own token count.
    """
    X = np.asarray(X, dtype=np.float64)
    B, H, L, d = X.shape
    bounds = block_bounds(L, b)
    out = np.empty((B, H, len(bounds), d), dtype=np.float64)
    for i, (lo, hi) in enumerate(bounds):
        out[:, :, i, :] = X[:, :, lo:hi, :].sum(axis=2) / (hi - lo)
    return out


# --------------------------------------------------------------------------
# O2  pooled scores
# --------------------------------------------------------------------------
def block_scores(Qbar, Kbar):
    """Pooled score S[b,h,i,j] = Qbar[b,h,i] . Kbar[b,h,j] (float64, unscaled).

    NEWS (efficient inference operators paragraph) says block relevance is
    judged from the current Q and K. Reading: the dot product of the block
    means, per (batch, head). Any positive scale or a row softmax is monotone
    and would pick the same blocks.
    """
    Qbar = np.asarray(Qbar, dtype=np.float64)
    Kbar = np.asarray(Kbar, dtype=np.float64)
    return np.matmul(Qbar, np.swapaxes(Kbar, -1, -2))


# --------------------------------------------------------------------------
# O3  how many key blocks each query block keeps
# --------------------------------------------------------------------------
def n_keep(nK: int, keep: float) -> int:
    """Number of key blocks kept per query block: min(nK, max(1, ceil(keep*nK - 1e-6))).

    NEWS and GUIDE give the kept share as 10-20 % of blocks (about 10 % for the
    INT8/FP8 kernel). Reading: every query-block row keeps the same count,
    the ceiling of keep*nK with keep held as a double; the 1e-6 guard stops a
    ratio such as 0.1 (not exact in binary) from rounding 192.00000000000003
    up to 193 at nK = 1920.
    """
    if not (0.0 < keep <= 1.0):
        raise ValueError("keep must be in (0, 1]")
    if nK < 1:
        raise ValueError("nK must be positive")
    return int(min(nK, max(1, math.ceil(float(keep) * nK - 1e-6))))


# --------------------------------------------------------------------------
# O4  per-row top-k selection
# --------------------------------------------------------------------------
def select_top_blocks(S, n: int):
    """Indices of the n largest scores of every row, ascending: int32 [..., n].

    NEWS: the important blocks are chosen at run time. Reading: a row keeps the
    n highest pooled scores; equal scores go to the lower block index; the kept
    indices are returned in ascending order, the order the tiles are visited.
    """
    S = np.asarray(S, dtype=np.float64)
    nK = S.shape[-1]
    if not (1 <= n <= nK):
        raise ValueError("n must be in [1, nK]")
    flat = S.reshape(-1, nK)
    idx = np.arange(nK)
    out = np.empty((flat.shape[0], n), dtype=np.int32)
    for r in range(flat.shape[0]):
        order = np.lexsort((idx, -flat[r]))  # by descending score, then ascending index
        out[r] = np.sort(order[:n])
    return out.reshape(S.shape[:-1] + (n,))


def plan(Q, K, bq: int, bk: int, keep: float):
    """Block plan [B, H, nQ, n_keep] (int32): O1 pool, O2 score, O3 count, O4 select."""
    Qbar = pool_block_means(Q, bq)
    Kbar = pool_block_means(K, bk)
    S = block_scores(Qbar, Kbar)
    return select_top_blocks(S, n_keep(Kbar.shape[2], keep))


# --------------------------------------------------------------------------
# O5  exact attention over the kept tiles
# --------------------------------------------------------------------------
def _kept_columns(plan_row, bounds_k):
    return np.concatenate([np.arange(*bounds_k[int(j)]) for j in plan_row])


def attend_exact(Q, K, V, plan_idx, bq: int, bk: int, sm=None, return_weights=False, rows=None):
    """Softmax attention of each query over the keys of its block's kept key blocks.

    NEWS (dynamic sparse quantized attention paragraph) and GUIDE (section 3):
    only the selected tiles are computed, densely inside each. Reading: no
    causal mask (video self-attention), softmax scale 1/sqrt(d) unless given,
    keys outside the kept blocks have weight zero. float64 throughout.
    With return_weights, also returns {(b,h,i): (columns, weights)}.
    rows: optional list of (b, h, i) query blocks to compute; others stay NaN.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, L, d = Q.shape
    sm = 1.0 / math.sqrt(d) if sm is None else float(sm)
    bq_bounds = block_bounds(L, bq)
    bk_bounds = block_bounds(L, bk)
    out = np.full(Q.shape, np.nan)
    weights = {}
    todo = rows if rows is not None else [
        (b, h, i) for b in range(B) for h in range(H) for i in range(len(bq_bounds))]
    for (b, h, i) in todo:
        r0, r1 = bq_bounds[i]
        cols = _kept_columns(plan_idx[b, h, i], bk_bounds)
        z = sm * (Q[b, h, r0:r1] @ K[b, h, cols].T)
        z -= z.max(axis=1, keepdims=True)
        w = np.exp(z)
        w /= w.sum(axis=1, keepdims=True)
        out[b, h, r0:r1] = w @ V[b, h, cols]
        if return_weights:
            weights[(b, h, i)] = (cols, w)
    return (out, weights) if return_weights else out


# --------------------------------------------------------------------------
# O6  brute force through a dense token mask (tiny inputs only)
# --------------------------------------------------------------------------
def attend_masked_dense(Q, K, V, plan_idx, bq: int, bk: int, sm=None):
    """Dense attention with M[n, m] = (key block of m is kept by query block of n).

    The same definition as attend_exact written the long way: a full L x L
    score matrix with the dropped entries set to -inf.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, L, d = Q.shape
    sm = 1.0 / math.sqrt(d) if sm is None else float(sm)
    out = np.empty_like(Q)
    for b in range(B):
        for h in range(H):
            M = np.zeros((L, L), dtype=bool)
            for n in range(L):
                kept = set(int(j) for j in plan_idx[b, h, n // bq])
                for m in range(L):
                    M[n, m] = (m // bk) in kept
            z = sm * (Q[b, h] @ K[b, h].T)
            z = np.where(M, z, -np.inf)
            z -= z.max(axis=1, keepdims=True)
            w = np.exp(z)
            w /= w.sum(axis=1, keepdims=True)
            out[b, h] = w @ V[b, h]
    return out


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------
def e4m3_rne(x):
    """Round float32 values with |x| <= 448 to OCP E4M3FN, ties to even (float32 result).

    E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; normals 2^(E-7)*(1+M/8),
    subnormals 2^-6*M/8, largest finite 448, no infinities. Values are rounded on
    the grid of their binade: step 2^(e-3) with e = max(floor(log2|x|), -6).
    """
    x = np.asarray(x, dtype=np.float32)
    ax = np.abs(x).astype(np.float64)
    if np.any(~np.isfinite(ax)) or np.any(ax > E4M3_MAX):
        raise ValueError("e4m3_rne takes finite values with |x| <= 448 (clamp first)")
    _, ex = np.frexp(ax)  # ax = f * 2^ex with f in [0.5, 1)
    e = np.maximum(ex - 1, -6)
    step = np.ldexp(1.0, e - 3)
    q = np.rint(ax / step) * step  # ax/step is exact (power-of-two step)
    return np.copysign(q, x).astype(np.float32)


def e4m3_bits(q):
    """Bit pattern (uint8) of values already on the E4M3FN grid."""
    q = np.asarray(q, dtype=np.float64)
    aq = np.abs(q)
    _, ex = np.frexp(aq)
    e = ex - 1
    normal = aq >= 2.0 ** -6
    E = np.where(normal, e + 7, 0)
    M = np.where(normal, (aq / np.ldexp(1.0, e) - 1.0) * 8.0, aq / 2.0 ** -9)
    if np.any(M != np.rint(M)) or np.any((E < 0) | (E > 15)):
        raise ValueError("value not on the E4M3FN grid")
    bits = (np.signbit(q).astype(np.uint8) << 7) | (E.astype(np.uint8) << 3) | M.astype(np.uint8)
    return bits.astype(np.uint8)


def e4m3_decode(bits):
    """Value (float32) of E4M3FN bit patterns; 0x7F/0xFF decode to NaN."""
    bits = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s = np.where(bits & 0x80, -1.0, 1.0)
    E = (bits >> 3) & 0xF
    M = bits & 0x7
    val = np.where(E == 0, M * 2.0 ** -9, np.ldexp(1.0 + M / 8.0, E - 7))
    val = np.where((E == 15) & (M == 7), np.nan, val)
    return (s * val).astype(np.float32)


def bf16_rne(x):
    """Round to bfloat16 (8 significant bits), ties to even, returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, ex = np.frexp(ax)
    e = np.maximum(ex - 1, -126)
    step = np.ldexp(1.0, e - 7)
    return np.copysign(np.rint(ax / step) * step, x)


# --------------------------------------------------------------------------
# Q1  per-block quantizers
# --------------------------------------------------------------------------
def _block_amax(X, lo, hi):
    return np.abs(X[:, :, lo:hi, :]).max(axis=(2, 3))  # float32 [B, H]


def quantize_int8_blocks(X, b: int):
    """Symmetric per-block INT8: returns (int8 [B,H,L,d], float32 scales [B,H,n]).

    NEWS (efficient inference operators paragraph) puts Q and K in INT8.
    Reading: one scale per (batch, head, block) over all d; a = max |x| over
    the block's valid tokens; s = a/127 and inv = 127/a, each one IEEE float32
    division (both 0 when a = 0); q = clamp(rint(float32(x*inv)), -127, 127),
    rint rounding ties to even. x ~ s*q.
    """
    X = np.asarray(X, dtype=np.float32)
    B, H, L, d = X.shape
    bounds = block_bounds(L, b)
    q = np.zeros(X.shape, dtype=np.int8)
    scales = np.zeros((B, H, len(bounds)), dtype=np.float32)
    f127 = np.float32(127.0)
    for i, (lo, hi) in enumerate(bounds):
        a = _block_amax(X, lo, hi)
        nz = a > 0
        safe = np.where(nz, a, np.float32(1.0)).astype(np.float32)
        s = np.where(nz, safe / f127, np.float32(0.0)).astype(np.float32)
        inv = np.where(nz, f127 / safe, np.float32(0.0)).astype(np.float32)
        y = (X[:, :, lo:hi, :] * inv[:, :, None, None]).astype(np.float32)
        q[:, :, lo:hi, :] = np.clip(np.rint(y), -127, 127).astype(np.int8)
        scales[:, :, i] = s
    return q, scales


def fp8_block_exponent(a):
    """Exponent e of a V block's power-of-two scale 2^e: the smallest integer with
    a <= 448 * 2^e, clamped to [-127, 127] (the range of an E8M0 scale); 0 when a = 0.

    With a = f * 2^k, f in [0.5, 1) (frexp) and 448 = 0.875 * 2^9: e = k - 9 if f <= 0.875,
    else k - 8. Exact for every float32 a.
    """
    a = np.asarray(a, dtype=np.float32)
    f, k = np.frexp(a)
    e = np.where(f <= np.float32(0.875), k - 9, k - 8)
    e = np.clip(e, -127, 127)
    return np.where(a > 0, e, 0).astype(np.int32)


def quantize_fp8_blocks(X, b: int):
    """Per-block FP8 E4M3FN: returns (float32 grid values [B,H,L,d], float32 scales [B,H,n]).

    NEWS (efficient inference operators paragraph) puts V in FP8 and leaves the scale open.
    Reading: OCP E4M3FN (largest finite 448), one power-of-two scale s = 2^e per
    (batch, head, block) with e = fp8_block_exponent(max |x| over the block): the block
    scale an MX-style (E8M0) FP8 operand carries, so the block's largest magnitude lands in
    (224, 448]; v = e4m3(clamp(float32(x * 2^-e), -448, 448)) rounded to nearest, ties to
    even (the power-of-two product is exact).
    """
    X = np.asarray(X, dtype=np.float32)
    B, H, L, d = X.shape
    bounds = block_bounds(L, b)
    q = np.zeros(X.shape, dtype=np.float32)
    scales = np.zeros((B, H, len(bounds)), dtype=np.float32)
    fmax = np.float32(E4M3_MAX)
    for i, (lo, hi) in enumerate(bounds):
        e = fp8_block_exponent(_block_amax(X, lo, hi)).astype(np.float64)
        s = np.exp2(e).astype(np.float32)
        inv = np.exp2(-e).astype(np.float32)
        y = (X[:, :, lo:hi, :] * inv[:, :, None, None]).astype(np.float32)
        q[:, :, lo:hi, :] = e4m3_rne(np.clip(y, -fmax, fmax))
        scales[:, :, i] = s
    return q, scales


# --------------------------------------------------------------------------
# Q2  tile-by-tile attention over INT8 Q/K and FP8 V
# --------------------------------------------------------------------------
def attend_quantized(Qh, sq, Kh, sk, Vq, sv, plan_idx, bq: int, bk: int, sm=None,
                     quantize_p: bool = True, rows=None):
    """Online-softmax attention over the kept tiles with INT8 Q/K and FP8 V.

    NEWS (efficient inference operators paragraph): the sparse kernel computes
    with Q/K in INT8 and V in FP8. Reading of the steps the pages leave open,
    for each query block i and each kept key block j in ascending order, taken
    as consecutive tiles of TILE_KEYS = 64 keys (a 128-key block is two tiles
    sharing the block's scales), with a running reference max m (an integer in
    the log2 domain, float32, starts at -inf), a row sum l and an accumulator
    acc (both carried in float64 here), per tile:
      S     = Qh_i . Kh_j^T, exact: integers (|S| <= 128*127^2 < 2^24) for INT8
              Q/K, or sums of 128 products of E4M3 values for FP8 Q/K (at most
              ~50 significant bits), so float64 BLAS is exact either way;
      g     = f32(f32(sq_i*sk_j) * f32(sm*log2 e));  x = f32(S*g)   (log2 domain)
      m'    = max(m, ceil(rowmax x));  alpha = 2^(m - m')  (exact; 0 while m = -inf)
      p     = f32(exp2(f32(x - m')))
      p8    = e4m3(f32(p * 2^8))              (p <= 1, so no saturation)
      l     = alpha*l + 2^-8 * sum p8         (the weights the PV product applies)
      acc   = alpha*acc + f32(sv_j * 2^-8) * (p8 . Vq_j)
    The reference max is the running max rounded up to an integer, so P's FP8
    scale 2^(8 - m') is a power of two (an E8M0 scale, like V's block scale).
    Finally O = acc / l (float64; the library rounds it to bf16). The row sum
    is taken over the FP8-rounded weights, the ones that multiply V, so the
    weights applied to V sum to one, as softmax attention's weights do: a
    constant V comes out unchanged.
    The all-FP8 path passes Q and K quantized by quantize_fp8_blocks (E4M3 grid
    values with power-of-two block scales) in place of the INT8 ones; the rest is
    the same.
    quantize_p=False keeps p8 = f32(p*2^8) unrounded (for the special-case pin).
    rows: optional list of (b, h, i) query blocks to compute; others stay NaN.
    """
    Qh = np.asarray(Qh)
    Kh = np.asarray(Kh)
    Vq = np.asarray(Vq, dtype=np.float32)
    B, H, L, d = Qh.shape
    sm = 1.0 / math.sqrt(d) if sm is None else float(sm)
    c = np.float32(sm * LOG2E)
    bq_bounds = block_bounds(L, bq)
    bk_bounds = block_bounds(L, bk)
    out = np.full((B, H, L, d), np.nan, dtype=np.float64)
    todo = rows if rows is not None else [
        (b, h, i) for b in range(B) for h in range(H) for i in range(len(bq_bounds))]
    for (b, h, i) in todo:
        r0, r1 = bq_bounds[i]
        qi = Qh[b, h, r0:r1].astype(np.float64)
        nr = r1 - r0
        m = np.full(nr, -np.inf, dtype=np.float32)
        l = np.zeros(nr, dtype=np.float64)
        acc = np.zeros((nr, d), dtype=np.float64)
        for j in sorted(int(t) for t in plan_idx[b, h, i]):
            b0, b1 = bk_bounds[j]
            g = np.float32(np.float32(sq[b, h, i] * sk[b, h, j]) * c)
            vs = np.float64(np.float32(sv[b, h, j] * np.float32(2.0 ** -8)))
            for c0 in range(b0, b1, TILE_KEYS):  # a kept block is visited as its 64-key tiles
                c1 = min(c0 + TILE_KEYS, b1)
                S = qi @ Kh[b, h, c0:c1].astype(np.float64).T
                x = (S.astype(np.float32) * g).astype(np.float32)
                m_new = np.maximum(m, np.ceil(x.max(axis=1)))
                alpha = np.exp2((m - m_new).astype(np.float64))  # a power of two (or 0)
                p = np.exp2((x - m_new[:, None]).astype(np.float64)).astype(np.float32)
                p8 = (p * np.float32(256.0)).astype(np.float32)
                if quantize_p:
                    p8 = e4m3_rne(p8)
                l = alpha * l + p8.sum(axis=1, dtype=np.float64) / 256.0
                acc = alpha[:, None] * acc + vs * (p8.astype(np.float64) @ Vq[b, h, c0:c1].astype(np.float64))
                m = m_new
        out[b, h, r0:r1] = acc / l[:, None]
    return out


# --------------------------------------------------------------------------
# Q3  how far the quantized path may land from exact attention
# --------------------------------------------------------------------------
def dequantize_blocks(Xq, s, b: int):
    """The values a block-quantized operand stands for: code * block scale (float64)."""
    Xq = np.asarray(Xq)
    out = np.empty(Xq.shape, dtype=np.float64)
    for i, (lo, hi) in enumerate(block_bounds(Xq.shape[2], b)):
        out[:, :, lo:hi] = Xq[:, :, lo:hi].astype(np.float64) * np.asarray(s, np.float64)[:, :, i, None, None]
    return out


def quantized_error_bound(Qh, sq, Kh, sk, Vq, sv, plan_idx, bq: int, bk: int, sm=None, rows=None,
                          score_rel_err: float = 0.0, out_bf16: bool = True):
    """Exact attention over the dequantized operands, and how far from it Q2's arithmetic
    (done in any order, in float32, with P rounded to E4M3) can land, per output element.

    The pages fix Q/K in INT8 and V in FP8 (NEWS, efficient inference operators
    paragraph) and say nothing of how P is carried; whatever the tile order, the
    reference-max policy or the float32 operation sequence, a path that rounds each
    weight of P to E4M3 (after a power-of-two scale) and normalises by the weights it
    applies lands within this bound of exact softmax attention over Qh*sq, Kh*sk,
    Vq*sv. Returns (exact, bound, rms), float64 [B, H, L, d], NaN outside `rows`:

      For a row, x_k = sm * log2(e) * (Qd . Kd_k) (log2 units), M = ceil(max x + e)
      the largest reference max the row can end on, P_k = 2^(x_k - M) <= 1, and
      O* = sum P V / sum P, the exact output.
      The path's weight for key k is P^_k (in units of 2^M) with
        |P^_k - P_k| <= d_k = (2^-4 (1 + n_k) + n_k) P_k + 2^-18
      where 2^-4 is E4M3's relative rounding error in its normal range, 2^-18 its
      subnormal spacing's half after the 2^8 pre-scale (in units of a reference max
      no larger than 2^M), and n_k = 2^(e_k) (1 + 2^-22) - 1 the relative error of
      the float32 exponential from a logit off by e_k:
        e_k = 2^-20 (|x_k| + |M| + 8) + g_k (1 + score_rel_err * A_k)
      (float32 rounding of the logit and of its offset by the reference max; one unit
      g_k = sq sk_k sm log2(e) of the integer score, which a conversion through a
      float32 offset may lose; for scores that are not exact, score_rel_err times
      A_k = sum_d |Qh_d Kh_kd| more).
      Since sum_k P_k (V_k - O*) = 0, the output with normalisation by the applied
      weights is off by sum_k (P^_k - P_k)(V_kc - O*_c) / sum P^, so
        |O_c - O*_c| <= t1 = sum_k d_k |V_kc - O*_c| / (sum P - sum d)
      plus 2^-10 of sum_k (P_k + d_k) |V_kc| / (sum P - sum d) and of |O*_c| + t1 for
      the float32 accumulation of P^ V and of the row sum (each 64-term product sum
      within 2^-10.9 of its largest term, each of up to ~2^11 tile sums added in float32),
      plus 2^-8 of the result for the bf16 output's rounding (out_bf16).
    rms is the expected size of the same difference when the rounding errors are
    independent and uniform over their grid steps (E4M3 step at P_k, bf16 step at O*).
    """
    Qh = np.asarray(Qh)
    Kh = np.asarray(Kh)
    B, H, L, d = Qh.shape
    sm = 1.0 / math.sqrt(d) if sm is None else float(sm)
    sq = np.asarray(sq, np.float64)
    sk = np.asarray(sk, np.float64)
    Qd = dequantize_blocks(Qh, sq, bq)
    Kd = dequantize_blocks(Kh, sk, bk)
    Vd = dequantize_blocks(Vq, sv, bk)
    bq_bounds = block_bounds(L, bq)
    bk_bounds = block_bounds(L, bk)
    key_blk = np.repeat(np.arange(len(bk_bounds)), [hi - lo for lo, hi in bk_bounds])
    exact = np.full((B, H, L, d), np.nan)
    bound = np.full((B, H, L, d), np.nan)
    rms = np.full((B, H, L, d), np.nan)
    todo = rows if rows is not None else [
        (b, h, i) for b in range(B) for h in range(H) for i in range(len(bq_bounds))]
    for (b, h, i) in todo:
        r0, r1 = bq_bounds[i]
        cols = _kept_columns(plan_idx[b, h, i], bk_bounds)
        x = (sm * LOG2E) * (Qd[b, h, r0:r1] @ Kd[b, h, cols].T)
        g = sq[b, h, i] * sk[b, h, key_blk[cols]] * (sm * LOG2E)
        e0 = 2.0 ** -20 * (np.abs(x) + 8.0) + g[None, :]
        if score_rel_err:
            A = np.abs(Qh[b, h, r0:r1].astype(np.float64)) @ np.abs(Kh[b, h, cols].astype(np.float64)).T
            e0 = e0 + g[None, :] * score_rel_err * A
        M = np.ceil((x + e0).max(axis=1, keepdims=True) + 2.0 ** -20 * (np.abs(x).max(axis=1, keepdims=True) + 9.0))
        e = e0 + 2.0 ** -20 * np.abs(M)
        M = np.maximum(M, np.ceil((x + e).max(axis=1, keepdims=True)))
        P = np.exp2(x - M)
        n = np.exp2(e) * (1.0 + 2.0 ** -22) - 1.0
        dk = (2.0 ** -4 * (1.0 + n) + n) * P + 2.0 ** -18
        V = Vd[b, h, cols]
        sP = P.sum(axis=1, keepdims=True)
        D = sP - dk.sum(axis=1, keepdims=True)
        O = (P @ V) / sP
        dev = np.abs(V[None, :, :] - O[:, None, :])  # [rows, keys, d]
        t1 = np.einsum("rk,rkc->rc", dk, dev) / D
        t2 = 2.0 ** -10 * (((P + dk) @ np.abs(V)) / D + np.abs(O) + t1)
        bd = t1 + t2
        if out_bf16:
            bd = bd + 2.0 ** -8 * (np.abs(O) + bd)
        bd = np.where(D > 0, bd, np.inf)
        # expected size: E4M3 step h at y = 2^8 P (normal from 2^-6, else the subnormal step)
        y = P * 256.0
        ey = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
        var_p = (np.exp2(ey - 3.0) / 256.0) ** 2 / 12.0
        var = np.einsum("rk,rkc->rc", var_p, dev ** 2) / sP ** 2
        if out_bf16:
            eo = np.floor(np.log2(np.maximum(np.abs(O), 2.0 ** -126)))
            var = var + np.exp2(eo - 7.0) ** 2 / 12.0
        exact[b, h, r0:r1] = O
        bound[b, h, r0:r1] = bd
        rms[b, h, r0:r1] = np.sqrt(var)
    return exact, bound, rms
