"""Pins of the CPU oracle to things other than itself (closed forms, library
routines, brute force, invariants, hand-worked examples). Runs on the CPU.

Each check is a function of the implementation it checks, so the same check is
also run on a copy of the oracle with a plausible mistake planted in it and
must fail there: that shows the pin would catch the mistake.
"""
import inspect
import json
import math
import os
import textwrap
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from oracle import blocksparse as ob

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def rng(seed=0):
    return np.random.default_rng(seed)


def planted(func, old, new):
    """A copy of an oracle function with one line of its source replaced (a planted
    mistake), compiled in the function's own module namespace."""
    src = textwrap.dedent(inspect.getsource(func))
    assert src.count(old) == 1, f"the text to replace occurs {src.count(old)} times"
    ns = dict(func.__globals__)
    exec(compile(src.replace(old, new), f"<planted {func.__name__}>", "exec"), ns)
    return ns[func.__name__]


# ---------------------------------------------------------------- O1 pooling
def check_pool_ramp(pool):
    # Q[n, c] = n + 1000 c: the mean of a block is its token midpoint (+1000 c),
    # a short last block included (L = 150, b = 64: blocks of 64, 64, 22 tokens).
    L, d = 150, 3
    X = (np.arange(L)[:, None] + 1000.0 * np.arange(d)[None, :])[None, None]
    got = pool(X, 64)
    mids = [31.5, 95.5, (128 + 149) / 2]
    want = np.array([[m + 1000.0 * c for c in range(d)] for m in mids])[None, None]
    assert got.shape == want.shape
    assert np.array_equal(got, want)


def check_pool_constant(pool):
    X = np.full((1, 2, 100, 4), 0.3, dtype=np.float32)
    got = pool(X, 64)
    assert np.array_equal(got, np.full((1, 2, 2, 4), np.float64(np.float32(0.3))))


def check_pool_bruteforce(pool):
    X = rng(1).standard_normal((2, 3, 37, 5))
    got = pool(X, 8)
    for b in range(2):
        for h in range(3):
            for i, lo in enumerate(range(0, 37, 8)):
                hi = min(lo + 8, 37)
                for c in range(5):
                    s = 0.0
                    for n in range(lo, hi):
                        s += X[b, h, n, c]
                    assert abs(got[b, h, i, c] - s / (hi - lo)) < 1e-14


def test_pool_pins():
    check_pool_ramp(oracle.pool_block_means)
    check_pool_constant(oracle.pool_block_means)
    check_pool_bruteforce(oracle.pool_block_means)


def test_pool_pin_catches_full_block_divisor():
    def bad(X, b):
        X = np.asarray(X, np.float64)
        bounds = ob.block_bounds(X.shape[2], b)
        return np.stack([X[:, :, lo:hi].sum(2) / b for lo, hi in bounds], axis=2)

    with pytest.raises(AssertionError):
        check_pool_ramp(bad)


def test_pool_matches_numpy_mean():
    X = rng(2).standard_normal((1, 2, 130, 16)).astype(np.float32)
    got = oracle.pool_block_means(X, 64)
    want = np.stack([X[:, :, lo:hi].astype(np.float64).mean(axis=2)
                     for lo, hi in [(0, 64), (64, 128), (128, 130)]], axis=2)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)


# ---------------------------------------------------------------- O2 scores
def check_scores(score):
    Qb = rng(3).standard_normal((1, 2, 3, 4))
    Kb = rng(4).standard_normal((1, 2, 5, 4))  # nQ != nK: a transposed product fails
    got = score(Qb, Kb)
    assert got.shape == (1, 2, 3, 5)
    want = torch.matmul(torch.from_numpy(Qb), torch.from_numpy(Kb).transpose(-1, -2)).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-14)
    for i in range(3):
        for j in range(5):
            s = sum(Qb[0, 1, i, c] * Kb[0, 1, j, c] for c in range(4))
            assert abs(got[0, 1, i, j] - s) < 1e-13


def test_scores_pin():
    check_scores(oracle.block_scores)


def test_scores_pin_catches_swapped_operands():
    with pytest.raises((AssertionError, ValueError)):
        check_scores(lambda Q, K: np.matmul(K, np.swapaxes(Q, -1, -2)))


# ---------------------------------------------------------------- O3 count
def test_n_keep_golden(golden_dir):
    with open(os.path.join(golden_dir, "n_keep.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        assert oracle.n_keep(c["nK"], c["keep"]) == c["n_keep"], c


def test_n_keep_closed_form_over_grid():
    # For ratios p/100 the exact ceiling is computable with rationals.
    for nK in (1, 2, 7, 16, 64, 512, 591, 1182, 1920):
        for pct in range(1, 101):
            exact = Fraction(pct, 100) * nK
            want = min(nK, max(1, math.ceil(exact)))
            assert oracle.n_keep(nK, pct / 100) == want, (nK, pct)


def test_n_keep_float32_trap_documented():
    # The trap the double-precision rule avoids: float32(0.1) widened overshoots.
    assert math.ceil(float(np.float32(0.1)) * 1920) == 193
    assert oracle.n_keep(1920, 0.1) == 192


def test_n_keep_rejects_bad_ratios():
    for bad in (0.0, -0.1, 1.5):
        with pytest.raises(ValueError):
            oracle.n_keep(10, bad)


# ---------------------------------------------------------------- O4 select
def brute_force_topk(row, n):
    # Repeatedly take the largest remaining score, lowest index among equals.
    left = list(range(len(row)))
    kept = []
    for _ in range(n):
        best = left[0]
        for j in left[1:]:
            if row[j] > row[best]:
                best = j
        kept.append(best)
        left.remove(best)
    return sorted(kept)


def check_select(select):
    r = rng(5)
    S = r.standard_normal((2, 3, 4, 19))
    S[0, 0, 0, 3] = S[0, 0, 0, 7] = S[0, 0, 0, 11] = 5.0  # forced ties at the top
    S[1, 2, 3, :] = 0.25  # a row of equal scores
    S[0, 1, 2, ::2] = S[0, 1, 2, 1]  # many ties
    for n in (1, 2, 5, 19):
        got = select(S, n)
        assert got.shape == (2, 3, 4, n)
        assert got.dtype == np.int32
        for b in range(2):
            for h in range(3):
                for i in range(4):
                    assert list(got[b, h, i]) == brute_force_topk(S[b, h, i], n), (b, h, i, n)


def test_select_pin():
    check_select(oracle.select_top_blocks)


def test_select_pin_catches_ties_to_higher_index():
    def bad(S, n):
        flat = S.reshape(-1, S.shape[-1])
        idx = np.arange(S.shape[-1])
        out = np.stack([np.sort(np.lexsort((-idx, -r))[:n]) for r in flat])
        return out.astype(np.int32).reshape(S.shape[:-1] + (n,))

    with pytest.raises(AssertionError):
        check_select(bad)


@settings(max_examples=60, deadline=None)
@given(nK=st.integers(1, 40), seed=st.integers(0, 10 ** 6), keep=st.floats(0.01, 1.0))
def test_select_properties(nK, seed, keep):
    r = np.random.default_rng(seed)
    row = np.round(r.standard_normal(nK), 1)  # rounding forces ties
    n = oracle.n_keep(nK, keep)
    got = oracle.select_top_blocks(row[None], n)[0]
    assert len(got) == n and list(got) == sorted(set(got.tolist()))
    dropped = [j for j in range(nK) if j not in set(got.tolist())]
    if dropped:
        kmin = min(row[got])
        assert kmin >= max(row[dropped])
        # every dropped block equal to the weakest kept one has a higher index
        for j in dropped:
            if row[j] == kmin:
                assert all(j > g for g in got if row[g] == kmin)


def test_select_keep_one_keeps_all():
    S = rng(6).standard_normal((1, 1, 3, 9))
    got = oracle.select_top_blocks(S, 9)
    assert np.array_equal(got, np.tile(np.arange(9, dtype=np.int32), (1, 1, 3, 1)))


def test_hand_examples(golden_dir):
    with open(os.path.join(golden_dir, "hand_examples.json")) as f:
        ex = json.load(f)["examples"]
    for e in ex:
        Q = np.array(e["Q"], np.float64)[None, None]
        K = np.array(e["K"], np.float64)[None, None]
        V = np.array(e["V"], np.float64)[None, None]
        Qb = oracle.pool_block_means(Q, e["bq"])
        Kb = oracle.pool_block_means(K, e["bk"])
        assert np.array_equal(Qb[0, 0], np.array(e["Qbar"], np.float64)), e["name"]
        assert np.array_equal(Kb[0, 0], np.array(e["Kbar"], np.float64)), e["name"]
        S = oracle.block_scores(Qb, Kb)
        assert np.array_equal(S[0, 0], np.array(e["S"], np.float64)), e["name"]
        p = oracle.plan(Q, K, e["bq"], e["bk"], e["keep"])
        assert p[0, 0].tolist() == e["plan"], e["name"]
        if "O" in e:
            O = oracle.attend_exact(Q, K, V, p, e["bq"], e["bk"])
            np.testing.assert_allclose(O[0, 0], np.array(e["O"], np.float64), rtol=0, atol=1e-14)


# ---------------------------------------------------------------- O5 / O6 attention
def _qkv(seed, B, H, L, d, scale=1.0):
    r = rng(seed)
    return tuple(scale * r.standard_normal((B, H, L, d)) for _ in range(3))


def check_attend_dense_at_keep_one(attend):
    Q, K, V = _qkv(7, 1, 2, 100, 16, 1.5)
    bq, bk = 32, 16
    nQ, nK = -(-100 // bq), -(-100 // bk)
    full = np.tile(np.arange(nK, dtype=np.int32), (1, 2, nQ, 1))
    got = attend(Q, K, V, full, bq, bk)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V)).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_attend_keep_one_equals_dense_sdpa():
    check_attend_dense_at_keep_one(oracle.attend_exact)


def test_attend_pin_catches_wrong_scale():
    def bad(Q, K, V, p, bq, bk):
        return oracle.attend_exact(Q, K, V, p, bq, bk, sm=1.0 / Q.shape[-1])

    with pytest.raises(AssertionError):
        check_attend_dense_at_keep_one(bad)


def check_attend_vs_masked(attend):
    Q, K, V = _qkv(8, 1, 2, 45, 8, 2.0)
    bq, bk = 16, 8
    p = oracle.plan(Q, K, bq, bk, 0.34)
    got = attend(Q, K, V, p, bq, bk)
    want = oracle.attend_masked_dense(Q, K, V, p, bq, bk)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_attend_matches_brute_force_mask():
    check_attend_vs_masked(oracle.attend_exact)


def test_attend_pin_catches_unapplied_plan():
    def bad(Q, K, V, p, bq, bk):  # attends to every key block, ignoring the plan
        nK = -(-Q.shape[2] // bk)
        full = np.broadcast_to(np.arange(nK, dtype=np.int32), p.shape[:3] + (nK,))
        return oracle.attend_exact(Q, K, V, full, bq, bk)

    with pytest.raises(AssertionError):
        check_attend_vs_masked(bad)


def test_attend_invariants():
    Q, K, V = _qkv(9, 1, 1, 70, 8, 2.0)
    bq, bk = 16, 8
    p = oracle.plan(Q, K, bq, bk, 0.3)
    O, W = oracle.attend_exact(Q, K, V, p, bq, bk, return_weights=True)
    for (_, _, _), (cols, w) in W.items():
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-13)
        assert np.all(w >= 0)
    # permuting each kept list leaves the output unchanged
    perm = p[..., ::-1].copy()
    np.testing.assert_allclose(oracle.attend_exact(Q, K, V, perm, bq, bk), O, rtol=0, atol=1e-12)
    # constant V gives a constant output
    Vc = np.full_like(V, -1.25)
    np.testing.assert_allclose(oracle.attend_exact(Q, K, Vc, p, bq, bk), -1.25, rtol=0, atol=1e-13)
    # Q = 0 gives the plain mean of V over the kept keys
    Oz = oracle.attend_exact(np.zeros_like(Q), K, V, p, bq, bk)
    bounds_k = ob.block_bounds(70, bk)
    for i, (r0, r1) in enumerate(ob.block_bounds(70, bq)):
        cols = np.concatenate([np.arange(*bounds_k[j]) for j in p[0, 0, i]])
        np.testing.assert_allclose(Oz[0, 0, r0:r1], np.broadcast_to(V[0, 0, cols].mean(0), (r1 - r0, 8)),
                                   rtol=0, atol=1e-13)


def test_attend_high_precision_tiny():
    # Two kept key blocks of one key each: the softmax by hand in
    # 50-digit arithmetic (mpmath), independent of numpy.
    import mpmath

    mpmath.mp.dps = 50
    Q = np.array([[[[0.3, -1.1], [5.0, 5.0], [-3.0, 1.0]]]])
    K = np.array([[[[1.0, 2.0], [-0.5, 0.25], [0.7, 0.7]]]])
    V = np.array([[[[1.0, -2.0], [3.0, 0.5], [9.0, 9.0]]]])
    pl = np.array([[[[0, 2]]]], np.int32)  # one query block of 3 tokens, keys 0 and 2
    got = oracle.attend_exact(Q, K, V, pl, 3, 1)
    sm = 1 / mpmath.sqrt(2)
    z = [sm * (mpmath.mpf(0.3) * K[0, 0, j, 0] + mpmath.mpf(-1.1) * K[0, 0, j, 1]) for j in (0, 2)]
    e = [mpmath.e ** zz for zz in z]
    for c in range(2):
        want = (e[0] * V[0, 0, 0, c] + e[1] * V[0, 0, 2, c]) / (e[0] + e[1])
        assert abs(got[0, 0, 0, c] - float(want)) < 1e-14


# ---------------------------------------------------------------- number formats
def _all_e4m3_values():
    bits = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_decode(bits)
    keep = ~np.isnan(vals)
    return bits[keep], vals[keep]


def check_e4m3(rne):
    bits, vals = _all_e4m3_values()
    pos = np.unique(vals[vals >= 0])
    mids = (pos[:-1] + pos[1:]) / 2  # exact ties: must go to the even mantissa
    r = rng(10)
    rand = np.concatenate([r.uniform(-448, 448, 20000), r.standard_normal(20000) * 0.02,
                           r.standard_normal(20000) * 2 ** -8])
    x = np.concatenate([pos, -pos, mids, -mids, rand]).astype(np.float32)
    got = rne(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(got, want)


def test_e4m3_matches_torch_cast():
    check_e4m3(oracle.e4m3_rne)


def test_e4m3_pin_catches_ties_away():
    def bad(x):
        x = np.asarray(x, np.float32)
        ax = np.abs(x).astype(np.float64)
        _, ex = np.frexp(ax)
        step = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3)
        return np.copysign(np.floor(ax / step + 0.5) * step, x).astype(np.float32)

    with pytest.raises(AssertionError):
        check_e4m3(bad)


def test_e4m3_codes_roundtrip_and_torch_bits():
    bits, vals = _all_e4m3_values()
    assert len(vals) == 254  # 256 codes minus the two NaNs
    assert vals.max() == 448.0 and np.min(np.abs(vals[vals != 0])) == 2.0 ** -9
    assert np.array_equal(oracle.e4m3_bits(vals)[vals != 0], bits[vals != 0])
    tb = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(tb[vals != 0], bits[vals != 0])


def test_e4m3_rejects_unclamped():
    with pytest.raises(ValueError):
        oracle.e4m3_rne(np.array([449.0], np.float32))


def test_bf16_rne_matches_torch():
    x = np.concatenate([rng(11).standard_normal(50000) * 3, rng(12).uniform(-1e3, 1e3, 50000)]).astype(np.float32)
    got = oracle.bf16_rne(x)
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- Q1 quantizers
def check_int8(quant):
    X = (rng(13).standard_normal((1, 2, 150, 16)) * 3).astype(np.float32)
    X[0, 1, 64:128] = 0.0  # an all-zero block
    X[0, 0, 140, 3] = 50.0  # the short last block gets its own scale
    q, s = quant(X, 64)
    assert q.dtype == np.int8 and s.dtype == np.float32 and s.shape == (1, 2, 3)
    assert s[0, 1, 1] == 0 and not q[0, 1, 64:128].any()
    assert s[0, 0, 2] == np.float32(np.float32(50.0) / np.float32(127.0))
    for h in range(2):
        for i, (lo, hi) in enumerate(ob.block_bounds(150, 64)):
            a = np.abs(X[0, h, lo:hi]).max()
            if a == 0:
                continue
            assert np.abs(q[0, h, lo:hi]).max() == 127
            err = np.abs(X[0, h, lo:hi].astype(np.float64) - s[0, h, i] * q[0, h, lo:hi])
            assert err.max() <= 0.5 * s[0, h, i] * (1 + 1e-5)
            inv = np.float32(127.0) / np.float32(a)
            y = X[0, h, lo:hi] * inv
            assert np.array_equal(q[0, h, lo:hi], torch.round(torch.from_numpy(y)).to(torch.int8).numpy())


def test_int8_quantizer_pins():
    check_int8(oracle.quantize_int8_blocks)


def test_int8_pin_catches_truncation():
    def bad(X, b):
        q, s = oracle.quantize_int8_blocks(X, b)
        inv = np.where(s > 0, np.float32(1) / np.where(s > 0, s, 1), 0)
        bounds = ob.block_bounds(X.shape[2], b)
        for i, (lo, hi) in enumerate(bounds):
            q[:, :, lo:hi] = np.trunc(X[:, :, lo:hi] * inv[:, :, i, None, None]).clip(-127, 127)
        return q, s

    with pytest.raises(AssertionError):
        check_int8(bad)


def test_int8_grid_inputs_are_identity():
    r = rng(14)
    X = r.integers(-127, 128, (1, 1, 128, 8)).astype(np.float32)
    X[0, 0, 5, 5] = 127.0
    X[0, 0, 70, 1] = -127.0
    q, s = oracle.quantize_int8_blocks(X, 64)
    assert np.array_equal(s, np.ones_like(s)) and np.array_equal(q, X.astype(np.int8))


def test_fp8_block_exponent_is_the_smallest_fitting_power():
    # Brute force in exact float64 arithmetic: e is the least integer with a <= 448 * 2^e.
    r = rng(21)
    a = np.concatenate([
        np.float32(448.0) * np.exp2(np.arange(-20, 21)).astype(np.float32),  # 448 * 2^k exactly
        np.nextafter(np.float32(448.0), np.float32(1e9)) * np.exp2(np.arange(-5, 6)).astype(np.float32),
        np.nextafter(np.float32(448.0), np.float32(0.0)) * np.exp2(np.arange(-5, 6)).astype(np.float32),
        np.float32(2.0) ** np.arange(-60, 60).astype(np.float32),
        (np.exp(r.uniform(-60, 60, 3000))).astype(np.float32),
    ]).astype(np.float32)
    e = oracle.fp8_block_exponent(a)
    a64 = a.astype(np.float64)
    assert np.all(a64 <= 448.0 * np.exp2(e.astype(np.float64)))
    assert np.all(a64 > 448.0 * np.exp2(e.astype(np.float64) - 1))
    # E8M0 range clamp and the all-zero block
    assert oracle.fp8_block_exponent(np.float32(3e38)) == 120
    assert oracle.fp8_block_exponent(np.float32(1e-45)) == -127
    assert oracle.fp8_block_exponent(np.float32(0.0)) == 0
    assert oracle.fp8_block_exponent(np.float32(448.0)) == 0
    assert oracle.fp8_block_exponent(np.float32(449.0)) == 1


def test_fp8_quantizer_pins():
    X = (rng(15).standard_normal((1, 2, 100, 16)) * 2).astype(np.float32)
    X[0, 1, :64] = 0
    X[0, 0, 64:] *= 1e3
    q, s = oracle.quantize_fp8_blocks(X, 64)
    assert s[0, 1, 0] == 1 and not q[0, 1, :64].any()
    for h in range(2):
        for i, (lo, hi) in enumerate(ob.block_bounds(100, 64)):
            a = np.abs(X[0, h, lo:hi]).max()
            if a == 0:
                continue
            e = np.log2(s[0, h, i])
            assert e == np.round(e)  # a power of two
            top = np.abs(q[0, h, lo:hi]).max()
            assert 224.0 <= top <= 448.0 and 224.0 < a / s[0, h, i] <= 448.0
            rel = np.abs(X[0, h, lo:hi] - s[0, h, i] * q[0, h, lo:hi]) / np.abs(X[0, h, lo:hi])
            normal = np.abs(q[0, h, lo:hi]) >= 2 ** -6
            assert rel[normal].max() <= 2.0 ** -4 * (1 + 1e-6)
            # the rounding itself against the library's e4m3 conversion
            y = X[0, h, lo:hi].astype(np.float64) / np.float64(s[0, h, i])
            assert np.array_equal(q[0, h, lo:hi], torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn).float().numpy())


def test_q2_128_key_block_is_two_64_key_tiles():
    # With equal block scales, a plan of 128-key blocks must give exactly what the plan of
    # their 64-key halves gives: the softmax state advances per 64-key tile either way.
    r = rng(23)
    L, d = 512, 16
    Qh = r.integers(-127, 128, (1, 1, L, d)).astype(np.float32)
    Kh = r.integers(-127, 128, (1, 1, L, d)).astype(np.float32)
    _, vals = _all_e4m3_values()
    Vq = r.choice(vals[np.abs(vals) <= 8], size=(1, 1, L, d)).astype(np.float32)
    sq = np.full((1, 1, 4), 0.01, np.float32)
    p128 = np.array([[[[0, 2], [1, 3], [2, 3], [0, 1]]]], np.int32)   # 4 query blocks of 128
    p64 = np.array([[[[0, 1, 4, 5], [2, 3, 6, 7], [4, 5, 6, 7], [0, 1, 2, 3]]]], np.int32)
    a = oracle.attend_quantized(Qh, sq, Kh, np.full((1, 1, 4), 0.02, np.float32), Vq,
                                np.full((1, 1, 4), 0.5, np.float32), p128, 128, 128)
    b = oracle.attend_quantized(Qh, sq, Kh, np.full((1, 1, 8), 0.02, np.float32), Vq,
                                np.full((1, 1, 8), 0.5, np.float32), p64, 128, 64)
    assert np.array_equal(a, b)


def test_fp8_grid_inputs_are_identity():
    _, vals = _all_e4m3_values()
    X = rng(16).choice(vals, size=(1, 1, 64, 16)).astype(np.float32)
    X[0, 0, 0, 0] = 448.0
    q, s = oracle.quantize_fp8_blocks(X, 64)
    assert s[0, 0, 0] == 1.0 and np.array_equal(q, X)


# ---------------------------------------------------------------- Q2 quantized attention
def _quantized_inputs(seed, L=200, d=16, bq=64, bk=32, keep=0.4):
    r = rng(seed)
    Q = (r.standard_normal((1, 2, L, d)) * 2).astype(np.float32)
    K = (r.standard_normal((1, 2, L, d)) * 2).astype(np.float32)
    V = r.standard_normal((1, 2, L, d)).astype(np.float32)
    p = oracle.plan(Q, K, bq, bk, keep)
    Qh, sq = oracle.quantize_int8_blocks(Q, bq)
    Kh, sk = oracle.quantize_int8_blocks(K, bk)
    Vq, sv = oracle.quantize_fp8_blocks(V, bk)
    return Qh, sq, Kh, sk, Vq, sv, p, bq, bk


def _dequant(Xq, s, b):
    out = np.zeros(Xq.shape, np.float64)
    for i, (lo, hi) in enumerate(ob.block_bounds(Xq.shape[2], b)):
        out[:, :, lo:hi] = Xq[:, :, lo:hi].astype(np.float64) * s[:, :, i, None, None]
    return out


def check_q2_unquantized_p(attend_q):
    Qh, sq, Kh, sk, Vq, sv, p, bq, bk = _quantized_inputs(17)
    got = attend_q(Qh, sq, Kh, sk, Vq, sv, p, bq, bk, quantize_p=False)
    want = oracle.attend_exact(_dequant(Qh, sq, bq), _dequant(Kh, sk, bk), _dequant(Vq, sv, bk), p, bq, bk)
    # Derived bound: x is rounded to float32 (|x| < 64 here, so < 4e-6 absolute
    # in the log2 domain) and the scale product g to float32; relative error
    # of the output stays below 1e-5.
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-5 * np.abs(want).max())


def test_q2_equals_exact_on_dequantized_without_p_rounding():
    check_q2_unquantized_p(oracle.attend_quantized)


def test_q2_pin_catches_missing_rescale():
    def bad(Qh, sq, Kh, sk, Vq, sv, p, bq, bk, quantize_p=True):
        # plants "acc is not multiplied by alpha" by running each tile on its own
        # max and summing the partial results without rescaling
        B, H, L, d = Qh.shape
        out = np.zeros((B, H, L, d))
        lsum = np.zeros((B, H, L, 1))
        for t in range(p.shape[-1]):
            pt = p[..., t:t + 1]
            o = oracle.attend_quantized(Qh, sq, Kh, sk, Vq, sv, pt, bq, bk, quantize_p=quantize_p)
            out += o
            lsum += 1
        return out / lsum

    with pytest.raises(AssertionError):
        check_q2_unquantized_p(bad)


def test_q2_p_rounding_within_fp8_bound():
    Qh, sq, Kh, sk, Vq, sv, p, bq, bk = _quantized_inputs(18)
    a = oracle.attend_quantized(Qh, sq, Kh, sk, Vq, sv, p, bq, bk, quantize_p=True)
    b = oracle.attend_quantized(Qh, sq, Kh, sk, Vq, sv, p, bq, bk, quantize_p=False)
    # Each weight moves by at most 2^-4 relative (normal E4M3) or 2^-10 absolute
    # after the 2^8 pre-scale (subnormal); bound |a - b| by the weighted |V|.
    vmax = np.abs(_dequant(Vq, sv, bk)).max()
    assert np.abs(a - b).max() <= (2.0 ** -4 + 2.0 ** -10 * 200) * vmax
    assert np.abs(a - b).max() > 0  # rounding did happen


def check_q2_applied_weights_sum_to_one(attend_q):
    """Softmax attention's weights sum to one over the keys a row attends to. In the
    quantized simulation the weights that multiply V are the FP8-rounded ones, so with V
    constant (per block, on the E4M3 grid after its power-of-two scale) every output is
    that constant, and with Q = 0 (every logit 0, every weight 1) every output is the
    plain mean of the dequantized V over the row's kept keys. Both hold for every query
    block, whatever the scores and the far-rescale steps of the other rows."""
    Qh, sq, Kh, sk, Vq, sv, p, bq, bk = _quantized_inputs(20)
    B, H, L, d = Qh.shape
    for c in (-1.25, 3.0, 0.7):  # 0.7 is not on the E4M3 grid: the output is its rounding
        Vc, svc = oracle.quantize_fp8_blocks(np.full((B, H, L, d), c, np.float32), bk)
        cq = float(Vc[0, 0, 0, 0]) * float(svc[0, 0, 0])
        assert (c != 0.7) == (cq == c)
        O = attend_q(Qh, sq, Kh, sk, Vc, svc, p, bq, bk)
        np.testing.assert_allclose(O, cq, rtol=1e-14, atol=0)
    Oz = attend_q(np.zeros_like(Qh), sq, Kh, sk, Vq, sv, p, bq, bk)
    Vd = _dequant(Vq, sv, bk)
    bounds_k = ob.block_bounds(L, bk)
    for h in range(H):
        for i, (r0, r1) in enumerate(ob.block_bounds(L, bq)):
            cols = np.concatenate([np.arange(*bounds_k[j]) for j in p[0, h, i]])
            want = np.broadcast_to(Vd[0, h, cols].mean(0), (r1 - r0, d))
            np.testing.assert_allclose(Oz[0, h, r0:r1], want, rtol=0, atol=1e-14)


def test_q2_applied_weights_sum_to_one():
    check_q2_applied_weights_sum_to_one(oracle.attend_quantized)


def test_q2_weights_pin_catches_row_sum_of_unrounded_p():
    # the earlier reading: the row sum over the float32 p before FP8 rounding
    bad = planted(ob.attend_quantized, "p8.sum(axis=1, dtype=np.float64) / 256.0",
                  "p.sum(axis=1, dtype=np.float64)")
    with pytest.raises(AssertionError):
        check_q2_applied_weights_sum_to_one(bad)


def test_q2_hand_example_equal_weights():
    # d = 2, L = 2, one block each. Inputs already on the grids, so every scale
    # is 1: Q rows (127, 0) and (0, 0); both keys (127, 0); V = diag(448).
    # sm = ln 2 makes sm * log2 e = 1, so the logits are the integers S (16129
    # and 0) and the reference max equals the row max. Within a row both keys
    # score the same, so p = 1 for both, p8 = 256,
    # acc = 2^-8 * 256 * (V0 + V1) = (448, 448) and l = 2: O = (224, 224).
    Q = np.array([[[[127, 0], [0, 0]]]], np.float32)
    K = np.array([[[[127, 0], [127, 0]]]], np.float32)
    V = np.array([[[[448, 0], [0, 448]]]], np.float32)
    Qh, sq = oracle.quantize_int8_blocks(Q, 2)
    Kh, sk = oracle.quantize_int8_blocks(K, 2)
    Vq, sv = oracle.quantize_fp8_blocks(V, 2)
    assert sq[0, 0, 0] == 1 and sk[0, 0, 0] == 1 and sv[0, 0, 0] == 1
    O = oracle.attend_quantized(Qh, sq, Kh, sk, Vq, sv, np.zeros((1, 1, 1, 1), np.int32), 2, 2,
                                sm=math.log(2.0))
    assert np.array_equal(O[0, 0], np.full((2, 2), 224.0))


def test_q2_reference_max_is_the_running_max_rounded_up():
    # One row, two keys with logits (in log2 units) 3.5 and 0.5 (sm = ln 2, S = 7/2 and 1/2
    # through the scales). The reference max is ceil(3.5) = 4, so p = (2^-0.5, 2^-3.5):
    # p8 = e4m3(2^7.5 = 181.02) = 176 and e4m3(2^4.5 = 22.63) = 22 (steps 16 and 2), and
    # O = (176 * 448 * 2^-8, 22 * 448 * 2^-8) / (2^-0.5 + 2^-3.5) over V = diag(448).
    # (A second query row of zeros scores 0 on both keys: O = (224, 224) as above.)
    Qh = np.array([[[[1, 0], [0, 0]]]], np.float32)
    Kh = np.array([[[[7, 0], [1, 0]]]], np.float32)
    Vq = np.array([[[[448, 0], [0, 448]]]], np.float32)
    one = np.ones((1, 1, 1), np.float32)
    O = oracle.attend_quantized(Qh, one * 0.5, Kh, one, Vq, one, np.zeros((1, 1, 1, 1), np.int32), 2, 2,
                                sm=math.log(2.0))
    # the row sum is that of the weights the PV product applies: (176 + 22) / 2^8
    l = (176.0 + 22.0) / 256
    want = np.array([176.0 * 448 / 256, 22.0 * 448 / 256]) / l
    np.testing.assert_allclose(O[0, 0, 0], want, rtol=1e-15)
    assert np.array_equal(O[0, 0, 1], [224.0, 224.0])


def test_q2_fp8_qk_reduces_to_exact_attention_on_dequantized_inputs():
    # All-FP8 path: Q and K on the E4M3 grid with power-of-two block scales. With P left
    # unrounded the tile-by-tile simulation must equal exact attention over the dequantized
    # Q, K, V (the scores are exact: sums of E4M3 products fit fp64).
    r = rng(31)
    L, d, bq, bk = 200, 16, 64, 32
    Q = (r.standard_normal((1, 2, L, d)) * 2).astype(np.float32)
    K = (r.standard_normal((1, 2, L, d)) * 2).astype(np.float32)
    V = r.standard_normal((1, 2, L, d)).astype(np.float32)
    p = oracle.plan(Q, K, bq, bk, 0.4)
    Qh, sq = oracle.quantize_fp8_blocks(Q, bq)
    Kh, sk = oracle.quantize_fp8_blocks(K, bk)
    Vq, sv = oracle.quantize_fp8_blocks(V, bk)
    got = oracle.attend_quantized(Qh, sq, Kh, sk, Vq, sv, p, bq, bk, quantize_p=False)
    want = oracle.attend_exact(_dequant(Qh, sq, bq), _dequant(Kh, sk, bk), _dequant(Vq, sv, bk), p, bq, bk)
    np.testing.assert_allclose(got, want, rtol=2e-5, atol=2e-6)
    # and the FP8 path's error against unquantized attention is that of 3-bit mantissas
    exact = oracle.attend_exact(Q, K, V, p, bq, bk)
    q8 = oracle.attend_quantized(Qh, sq, Kh, sk, Vq, sv, p, bq, bk)
    assert 1e-3 < np.linalg.norm(q8 - exact) / np.linalg.norm(exact) < 0.2


def test_q2_rows_subset_matches_full():
    Qh, sq, Kh, sk, Vq, sv, p, bq, bk = _quantized_inputs(19)
    full = oracle.attend_quantized(Qh, sq, Kh, sk, Vq, sv, p, bq, bk)
    part = oracle.attend_quantized(Qh, sq, Kh, sk, Vq, sv, p, bq, bk, rows=[(0, 1, 2)])
    np.testing.assert_array_equal(part[0, 1, 128:192], full[0, 1, 128:192])
    assert np.isnan(part[0, 0]).all()


# ---------------------------------------------------------------- Q3 bound against exact attention
def _q3_cases():
    yield "rand", _quantized_inputs(17)
    yield "ragged", _quantized_inputs(21, L=157, d=8, bq=32, bk=64, keep=0.5)
    # rows whose max rises far after their first kept block (exercises the rescale steps)
    r = rng(22)
    L, d, bq, bk = 192, 16, 64, 32
    u = np.full(d, 0.5)
    Q = (u + 0.3 * r.standard_normal((1, 1, L, d))).astype(np.float32) * 3
    K = (u + 0.3 * r.standard_normal((1, 1, L, d))).astype(np.float32) * 3
    K[:, :, -bk:] *= 6
    V = r.standard_normal((1, 1, L, d)).astype(np.float32)
    p = oracle.plan(Q, K, bq, bk, 0.5)
    Qh, sq = oracle.quantize_int8_blocks(Q, bq)
    Kh, sk = oracle.quantize_int8_blocks(K, bk)
    Vq, sv = oracle.quantize_fp8_blocks(V, bk)
    yield "far", (Qh, sq, Kh, sk, Vq, sv, p, bq, bk)


def check_q3_exact(bound_fn):
    for _, (Qh, sq, Kh, sk, Vq, sv, p, bq, bk) in _q3_cases():
        ex, _, _ = bound_fn(Qh, sq, Kh, sk, Vq, sv, p, bq, bk)
        want = oracle.attend_exact(_dequant(Qh, sq, bq), _dequant(Kh, sk, bk), _dequant(Vq, sv, bk), p, bq, bk)
        np.testing.assert_allclose(ex, want, rtol=0, atol=1e-13)


def test_q3_exact_is_exact_attention_on_dequantized_operands():
    check_q3_exact(oracle.quantized_error_bound)


def test_q3_exact_pin_catches_missing_log2e():
    bad = planted(ob.quantized_error_bound, "x = (sm * LOG2E) * (", "x = sm * (")
    with pytest.raises(AssertionError):
        check_q3_exact(bad)


def check_q3_bound_holds(bound_fn):
    """The quantized simulation (one way of doing the arithmetic), rounded to bf16, lands
    within the bound everywhere, and its error is the predicted size (within 15 %)."""
    for name, (Qh, sq, Kh, sk, Vq, sv, p, bq, bk) in _q3_cases():
        ex, bd, rms = bound_fn(Qh, sq, Kh, sk, Vq, sv, p, bq, bk)
        got = oracle.bf16_rne(oracle.attend_quantized(Qh, sq, Kh, sk, Vq, sv, p, bq, bk))
        assert np.all(np.abs(got - ex) <= bd), name
        ratio = np.linalg.norm(got - ex) / np.linalg.norm(rms)
        assert 0.85 <= ratio <= 1.15, (name, ratio)


def test_q3_bound_holds_for_the_quantized_simulation():
    check_q3_bound_holds(oracle.quantized_error_bound)


def test_q3_bound_pin_catches_missing_fp8_term():
    bad = planted(ob.quantized_error_bound, "dk = (2.0 ** -4 * (1.0 + n) + n) * P", "dk = n * P")
    with pytest.raises(AssertionError):
        check_q3_bound_holds(bad)


def test_q3_rms_pin_catches_step_of_the_wrong_binade():
    bad = planted(ob.quantized_error_bound, "var_p = (np.exp2(ey - 3.0)", "var_p = (np.exp2(ey - 2.0)")
    with pytest.raises(AssertionError):
        check_q3_bound_holds(bad)


def test_q3_first_term_is_the_worst_case_over_weight_perturbations():
    """Brute force: for a row of 7 keys, every output obtained by moving each weight P_k
    anywhere within +-d_k (all 2^7 corners of that box, where the extremes lie, and random
    interior points) stays within t1 = sum d_k |V_k - O*| / (sum P - sum d), and the
    worst corner comes within a factor (sum P - sum d)/(sum P + sum d) of it."""
    r = rng(23)
    P = r.uniform(0.05, 1.0, 7)
    V = r.standard_normal(7)
    dk = 2.0 ** -4 * P + 2.0 ** -18
    O = (P @ V) / P.sum()
    t1 = (dk @ np.abs(V - O)) / (P.sum() - dk.sum())
    worst = 0.0
    for corner in range(2 ** 7):
        s = np.array([1.0 if corner >> k & 1 else -1.0 for k in range(7)])
        Ph = P + s * dk
        worst = max(worst, abs((Ph @ V) / Ph.sum() - O))
    for _ in range(2000):
        Ph = P + r.uniform(-1, 1, 7) * dk
        assert abs((Ph @ V) / Ph.sum() - O) <= t1 * (1 + 1e-12)
    assert worst <= t1 * (1 + 1e-12)
    assert worst >= t1 * (P.sum() - dk.sum()) / (P.sum() + dk.sum()) * (1 - 1e-12)


def test_q3_bound_is_reached_in_part_by_a_constructed_row():
    """Two queries, two keys of one token each (block_k = 1), d = 1, sm = ln 2 so logits are
    integer scores times the scales. Query 0 scores 0 on key 0 and -s on key 1, with
    s = -log2(136/256 (1 - 2^-20)): p * 2^8 is 256 for key 0 (exact in E4M3) and
    136 (1 - 2^-20) for key 1, just below the midpoint of E4M3's 128 and 144, so it rounds
    down by 5.9 % (E4M3's largest relative step is 6.25 %). With V = (1, -1) that whole move
    reaches the output: O = (256 - 128) / (256 + 128) = 1/3 against the exact
    (1 - r) / (1 + r), r = 136/256 (1 - 2^-20), and the bound must hold with no more than
    2.5 times the distance (the bound also covers key 0 moving by 6.25 %). Query 1 is all
    zero: equal weights, O = 0 on both sides."""
    r = 136.0 / 256.0 * (1.0 - 2.0 ** -20)
    Qh = np.array([[[[127], [0]]]], np.int8)
    Kh = np.array([[[[0], [-127]]]], np.int8)
    sq = np.ones((1, 1, 1), np.float32)
    sk = np.full((1, 1, 2), -math.log2(r) / 127 ** 2, np.float32)
    Vq = np.array([[[[256.0], [-256.0]]]], np.float32)
    sv = np.full((1, 1, 2), 2.0 ** -8, np.float32)
    p = np.array([[[[0, 1]]]], np.int32)
    args = (Qh, sq, Kh, sk, Vq, sv, p, 2, 1)
    ex, bd, _ = oracle.quantized_error_bound(*args, sm=math.log(2.0))
    got = oracle.attend_quantized(*args, sm=math.log(2.0))
    assert got[0, 0, 0, 0] == 1.0 / 3.0 and got[0, 0, 1, 0] == 0.0
    np.testing.assert_allclose(ex[0, 0, 0, 0], (1 - r) / (1 + r), rtol=1e-6)
    moved = abs(got[0, 0, 0, 0] - ex[0, 0, 0, 0])
    assert bd[0, 0, 0, 0] / 2.5 <= moved <= bd[0, 0, 0, 0]


# ---------------------------------------------------------------- Light-Ulysses FP8 packing
def test_ulysses_rows_quantize_like_the_library_e4m3_cast():
    from oracle import ulysses as uo
    r = rng(41)
    x = (r.standard_normal((2, 3, 50, 128)) * np.exp(r.uniform(-8, 8, (2, 3, 50, 1)))).astype(np.float32)
    x[0, 0, 0] = 0.0
    q, e = uo.fp8_rows(x)
    assert e[0, 0, 0] == 0 and not q[0, 0, 0].any()
    a = np.abs(x).max(-1)
    nz = a > 0
    assert np.all((a[nz] <= 448.0 * np.exp2(e[nz].astype(np.float64))) & (a[nz] > 224.0 * np.exp2(e[nz].astype(np.float64))))
    y = (x.astype(np.float64) * np.exp2(-e.astype(np.float64))[..., None]).astype(np.float32)
    lib = torch.from_numpy(y).to(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(q, lib)


def test_ulysses_exchange_round_trip_is_one_quantization():
    # seq -> head -> (identity attention) -> head -> seq gives every row quantized once more,
    # and re-quantizing a row already on the grid changes nothing (its exponent stays).
    from oracle import ulysses as uo
    r = rng(42)
    B, H, L, d, P = 1, 8, 103, 16, 4
    x = (r.standard_normal((B, H, L, d)) * 3).astype(np.float32)
    per_peer = uo.seq_to_head([x], P)
    assert [t[0].shape for t in per_peer] == [(B, H // P, L, d)] * P
    back = uo.head_to_seq([t[0].astype(np.float32) for t in per_peer], L, P)
    bounds, lmax = uo.shard_bounds(L, P)
    assert lmax == 26 and bounds[-1] == (78, 103)
    once = uo.dequant_rows(x)
    for (lo, hi), y in zip(bounds, back):
        assert np.array_equal(y, once[:, :, lo:hi])


def test_ulysses_payload_layout_by_loops():
    from oracle import ulysses as uo
    r = rng(43)
    B, H, L, d, P, rank = 2, 4, 10, 8, 2, 1
    full = [(r.standard_normal((B, H, L, d)) * 2).astype(np.float32) for _ in range(3)]
    bounds, lmax = uo.shard_bounds(L, P)
    lo, hi = bounds[rank]
    local = [t[:, :, lo:hi] for t in full]
    codes, exps = uo.payload(local, L, rank, P)
    assert codes.shape == (P, B, lmax, H // P, 3, d)
    for p in range(P):
        for b in range(B):
            for t in range(lmax):
                for hh in range(H // P):
                    for ti in range(3):
                        if lo + t >= hi:
                            assert not codes[p, b, t, hh, ti].any() and exps[p, b, t, hh, ti] == 0
                            continue
                        row = local[ti][b, p * (H // P) + hh, t]
                        q, e = uo.fp8_rows(row[None])
                        assert np.array_equal(codes[p, b, t, hh, ti], q[0]) and exps[p, b, t, hh, ti] == e[0]


def test_ulysses_head_chunk_payload_by_loops():
    # a head chunk of every group, and the way back from the head split, slot by slot
    from oracle import ulysses as uo
    r = rng(44)
    B, H, L, d, P, rank, h0, hc = 1, 6, 7, 4, 3, 2, 1, 1
    full = [(r.standard_normal((B, H, L, d)) * 5).astype(np.float32) for _ in range(2)]
    bounds, lmax = uo.shard_bounds(L, P)
    assert lmax == 3 and bounds == [(0, 3), (3, 6), (6, 7)]
    lo, hi = bounds[rank]
    codes, exps = uo.payload([t[:, :, lo:hi] for t in full], L, rank, P, h0, hc)
    assert codes.shape == (P, B, lmax, hc, 2, d)
    for p in range(P):
        for t in range(lmax):
            for ti in range(2):
                if lo + t >= hi:
                    assert not codes[p, 0, t, 0, ti].any() and exps[p, 0, t, 0, ti] == 0
                    continue
                q, e = uo.fp8_rows(full[ti][0, p * (H // P) + h0, lo + t][None])
                assert np.array_equal(codes[p, 0, t, 0, ti], q[0]) and exps[p, 0, t, 0, ti] == e[0]
    heads = [t[:, 2:4] for t in full]  # a peer's [B, hc=2, L, d] chunk on the way back
    codes, exps = uo.payload_back(heads, P)
    assert codes.shape == (P, B, lmax, 2, 2, d)
    for p, (a, b) in enumerate(bounds):
        for t in range(lmax):
            for hh in range(2):
                for ti in range(2):
                    if a + t >= b:
                        assert not codes[p, 0, t, hh, ti].any() and exps[p, 0, t, hh, ti] == 0
                        continue
                    q, e = uo.fp8_rows(heads[ti][0, hh, a + t][None])
                    assert np.array_equal(codes[p, 0, t, hh, ti], q[0]) and exps[p, 0, t, hh, ti] == e[0]


# ---------------------------------------------------------------- Q/K prologue (RMSNorm, 3-D RoPE)
def check_rmsnorm_torch(fn, rtol):
    r = rng(51)
    X = (r.standard_normal((2, 3, 17, 128)) * r.uniform(0.1, 10, (2, 3, 17, 1))).astype(np.float32)
    g = r.uniform(0.5, 1.5, (3, 128)).astype(np.float32)
    got = fn(X, g, 1e-6)
    for h in range(3):
        want = torch.nn.functional.rms_norm(torch.from_numpy(X[:, h]).double(), (128,),
                                            weight=torch.from_numpy(g[h]).double(), eps=1e-6).numpy()
        assert np.allclose(got[:, h], want, rtol=rtol, atol=0)


def check_rmsnorm_constant_row(fn, rtol):
    # a row of equal values c: mean square c^2, so y = c / sqrt(c^2 + eps) * g
    X = np.full((1, 1, 1, 8), 0.25)
    g = np.arange(1, 9, dtype=np.float64)[None]
    got = fn(X, g, 0.0625)
    assert np.allclose(got[0, 0, 0], 0.25 / math.sqrt(0.0625 + 0.0625) * np.arange(1, 9), rtol=rtol)


def test_rmsnorm_pins():
    from oracle import prologue as po
    check_rmsnorm_torch(po.rms_norm64, 1e-13)
    check_rmsnorm_constant_row(po.rms_norm64, 1e-15)
    # the fp32 operations: within a few fp32 rounding steps of the fp64 definition
    check_rmsnorm_torch(po.rms_norm, 4 * 2.0 ** -24)
    check_rmsnorm_constant_row(po.rms_norm, 4 * 2.0 ** -24)


def test_rmsnorm_fp32_steps_are_ieee_operations():
    # each step is one rounded fp32 operation: recompute one row by hand with Python floats
    from oracle import prologue as po
    r = rng(55)
    x = torch.from_numpy(r.standard_normal(128).astype(np.float32)).bfloat16().float().numpy()
    g = r.uniform(0.5, 1.5, 128).astype(np.float32)
    got = po.rms_norm(x[None, None, None], g[None], 1e-6)[0, 0, 0]
    ss = math.fsum(float(v) * float(v) for v in x)  # exact
    f32 = lambda v: float(np.float32(v))
    rr = f32(1.0 / f32(math.sqrt(f32(f32(ss / 128) + f32(1e-6)))))
    want = np.array([f32(f32(float(v) * rr) * float(gg)) for v, gg in zip(x, g)], np.float32)
    assert np.array_equal(got, want)


def test_rmsnorm_pins_catch_missing_eps_and_wrong_axis():
    def no_eps(X, g, eps):
        X = np.asarray(X, np.float64)
        return X / np.sqrt(np.mean(X * X, axis=-1, keepdims=True)) * np.asarray(g)[None, :, None, :]

    def over_tokens(X, g, eps):
        X = np.asarray(X, np.float64)
        return X / np.sqrt(np.mean(X * X, axis=-2, keepdims=True) + eps) * np.asarray(g)[None, :, None, :]

    with pytest.raises(AssertionError):
        check_rmsnorm_constant_row(no_eps, 1e-6)
    with pytest.raises(AssertionError):
        check_rmsnorm_torch(over_tokens, 1e-6)


def check_rope_complex(fn):
    # Brute force with complex numbers, token by token: channel pair p is the complex number
    # x_2p + i x_2p+1, multiplied by exp(i * pos * 10000^(-j/n)) for its axis group.
    grid = (3, 4, 5)
    L, d = 60, 128
    X = rng(52).standard_normal((1, 2, L, d))
    got = fn(X, grid)
    groups = [("t", 22), ("y", 21), ("x", 21)]
    for h in range(2):
        for n in range(L):
            t, rest = divmod(n, 4 * 5)
            y, x = divmod(rest, 5)
            pos = {"t": t, "y": y, "x": x}
            p = 0
            for axis, cnt in groups:
                for j in range(cnt):
                    z = complex(X[0, h, n, 2 * p], X[0, h, n, 2 * p + 1])
                    w = z * complex(math.cos(pos[axis] * 10000.0 ** (-j / cnt)),
                                    math.sin(pos[axis] * 10000.0 ** (-j / cnt)))
                    tol = 5e-7 * (abs(z.real) + abs(z.imag) + 1e-30)  # fp32 steps
                    assert abs(got[0, h, n, 2 * p] - w.real) <= tol and abs(got[0, h, n, 2 * p + 1] - w.imag) <= tol
                    p += 1


def check_rope_hand(fn):
    # d = 6: one pair per axis, each turning by its coordinate (10000^0 = 1) on a 2x2x2 grid.
    X = np.tile(np.array([1.0, 0.0, 0.0, 1.0, 2.0, 3.0]), (1, 1, 8, 1))
    got = fn(X, (2, 2, 2))
    c, s = math.cos(1.0), math.sin(1.0)
    assert np.array_equal(got[0, 0, 0], X[0, 0, 0])  # token 0 = (0, 0, 0): identity
    tol = 1e-6
    assert np.allclose(got[0, 0, 1], [1, 0, 0, 1, 2 * c - 3 * s, 2 * s + 3 * c], rtol=0, atol=tol)  # (0,0,1)
    assert np.allclose(got[0, 0, 2], [1, 0, -s, c, 2, 3], rtol=0, atol=tol)  # (0, 1, 0)
    assert np.allclose(got[0, 0, 7], [c, s, -s, c, 2 * c - 3 * s, 2 * s + 3 * c], rtol=0, atol=tol)


def check_rope_relative(fn):
    # The score of a rotated q at token n with a rotated k at token m depends only on the
    # coordinate differences: tokens shifted together by (1, 1, 1) give the same score.
    grid = (4, 4, 4)
    d = 128
    r = rng(53)
    q, k = r.standard_normal(d), r.standard_normal(d)
    Q = fn(np.tile(q, (1, 1, 64, 1)), grid)[0, 0]
    K = fn(np.tile(k, (1, 1, 64, 1)), grid)[0, 0]
    tok = lambda t, y, x: (t * 4 + y) * 4 + x
    a = Q[tok(0, 1, 2)] @ K[tok(2, 0, 1)]
    b = Q[tok(1, 2, 3)] @ K[tok(3, 1, 2)]
    assert abs(a - b) <= 1e-5 * np.abs(q).sum() * np.abs(k).sum() / d
    assert np.allclose(np.linalg.norm(Q, axis=-1), np.linalg.norm(q), rtol=1e-6)


def test_rope_pins():
    from oracle import prologue as po
    assert po.axis_pairs(128) == (22, 21, 21) and po.axis_pairs(6) == (1, 1, 1)
    for fn in (po.rope3d, po.rope3d64):
        check_rope_complex(fn)
        check_rope_hand(fn)
        check_rope_relative(fn)


def test_rope_pins_catch_half_split_pairs_and_swapped_axes():
    from oracle import prologue as po

    def half_split(X, grid, theta=10000.0):  # pairs (i, i + d/2) instead of adjacent channels
        X = np.asarray(X, np.float64)
        L, d = X.shape[2], X.shape[3]
        c, s = po.rope_cos_sin(grid, L, d, theta)
        c, s = c.astype(np.float64)[None, None], s.astype(np.float64)[None, None]
        x0, x1 = X[..., :d // 2], X[..., d // 2:]
        return np.concatenate([x0 * c - x1 * s, x0 * s + x1 * c], axis=-1)

    def swapped_axes(X, grid, theta=10000.0):  # column axis first
        T, Hg, Wg = grid
        X = np.asarray(X, np.float64)
        L, d = X.shape[2], X.shape[3]
        n = np.arange(L)
        pos = (n % Wg, (n // Wg) % Hg, n // (Hg * Wg))
        ang = np.concatenate([p[:, None] * theta ** (-np.arange(m) / m)[None, :]
                              for p, m in zip(pos, po.axis_pairs(d))], axis=1)
        c, s = np.cos(ang)[None, None], np.sin(ang)[None, None]
        out = np.empty_like(X)
        out[..., 0::2] = X[..., 0::2] * c - X[..., 1::2] * s
        out[..., 1::2] = X[..., 0::2] * s + X[..., 1::2] * c
        return out

    with pytest.raises(AssertionError):
        check_rope_complex(half_split)
    with pytest.raises(AssertionError):
        check_rope_complex(swapped_axes)
    with pytest.raises(AssertionError):
        check_rope_hand(swapped_axes)


def test_prologue_is_norm_then_rope_in_fp32_steps():
    from oracle import prologue as po
    r = rng(54)
    X = torch.from_numpy(r.standard_normal((1, 2, 40, 128)).astype(np.float32)).bfloat16().float().numpy()
    g = r.uniform(0.5, 2.0, (2, 128)).astype(np.float32)
    got = po.qk_prologue(X, g, 1e-6, (2, 4, 5))
    assert got.dtype == np.float32
    assert np.array_equal(got, po.rope3d(po.rms_norm(X, g, 1e-6), (2, 4, 5)))
    # within fp32's error bound of the fp64 definition (per pair: a few rounding steps of |x0|+|x1|)
    exact = po.rope3d64(po.rms_norm64(X, g, 1e-6), (2, 4, 5))
    pair = np.abs(exact[..., 0::2]) + np.abs(exact[..., 1::2])
    bound = 8 * 2.0 ** -24 * np.repeat(pair, 2, axis=-1)
    assert np.all(np.abs(got - exact) <= bound)
    Y64, b64 = po.qk_prologue64(X, g, 1e-6, (2, 4, 5))
    assert np.array_equal(Y64, exact) and np.array_equal(b64, bound)
    # the bound is not loose by orders of magnitude: the largest deviation uses a good part of it
    assert (np.abs(got - exact) / bound).max() > 0.05
    # rotation keeps each pair's length, so the normalized row's mean square (g = 1) stays 1
    ones = po.qk_prologue(X, np.ones((2, 128), np.float32), 0.0, (2, 4, 5)).astype(np.float64)
    assert np.allclose(np.mean(ones * ones, axis=-1), 1.0, rtol=1e-6)


# ---------------------------------------------------------------- NVFP4 block-scaled GEMM
def _e2m1_by_thresholds(v):
    # RNE onto {0, .5, 1, 1.5, 2, 3, 4, 6} written as threshold counting: a midpoint goes to the
    # neighbour with the even mantissa bit (codes 0, 2, 4, 6), so the comparison is '>' below an
    # even code and '>=' below an odd one... restated per midpoint: 0.25 -> 0, 0.75 -> 1,
    # 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4.
    a = abs(float(v))
    idx = (a > 0.25) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) + (a > 5.0)
    val = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0][idx]
    return -val if math.copysign(1.0, v) < 0 else val


def check_e2m1(fn):
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = [0.0, -0.0, 6.0, 7.0, 1e30, -1e30, 0.1, -0.1, 5.999, 6.001]
    for m in mids:
        for d in (-1e-6, 0.0, 1e-6):
            vals += [m + d, -(m + d)]
    vals += list(rng(61).uniform(-8, 8, 4000))
    v = np.array(vals, np.float32)
    got = fn(v)
    want = np.array([_e2m1_by_thresholds(x) for x in v], np.float32)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_e2m1_pins():
    from oracle import nvfp4 as nf
    check_e2m1(nf.e2m1_rne)
    q = nf.e2m1_rne(np.array([0.5, -6.0, 1.5, -0.0], np.float32))
    assert nf.e2m1_bits(q).tolist() == [1, 15, 3, 8]


def test_e2m1_pin_catches_ties_away_from_zero():
    def away(v):
        a = np.abs(np.asarray(v, np.float64))
        grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
        d = np.abs(a[..., None] - grid)
        idx = np.where(a > 6, 7, 7 - np.argmin(d[..., ::-1], axis=-1))  # ties to the larger value
        return np.where(np.signbit(v), -grid[idx], grid[idx]).astype(np.float32)

    with pytest.raises(AssertionError):
        check_e2m1(away)


def check_nvfp4_hand(quantize):
    # one block 0..15: amax 15, S = 15/2688, s = e4m3(15 / (6 S)) = 448, x / (448 S) = x / 2.5
    X = np.arange(16, dtype=np.float32)[None]
    q, s, S = quantize(X)
    assert np.float32(S) == np.float32(np.float32(15) / np.float32(2688))
    assert s.shape == (1, 1) and s[0, 0] == 448.0
    assert q[0].tolist() == [0, 0.5, 1, 1, 1.5, 2, 2, 3, 3, 4, 4, 4, 4, 6, 6, 6]


def check_nvfp4_blocks_along_k(quantize):
    # two rows, two blocks each, very different magnitudes: every (row, 16-block) has its own scale
    X = np.zeros((2, 32), np.float32)
    X[0, :16], X[0, 16:], X[1, :16], X[1, 16:] = 1.0, 100.0, 0.1, 3000.0
    q, s, S = quantize(X)
    assert np.float32(S) == np.float32(np.float32(3000) / np.float32(2688))
    assert s.shape == (2, 2)
    deq = q.astype(np.float64).reshape(2, 2, 16) * s[..., None] * S
    assert np.allclose(deq.reshape(2, 32), X, rtol=0.07)  # each block's own scale keeps it within E2M1 steps


def test_nvfp4_quantize_pins():
    from oracle import nvfp4 as nf
    check_nvfp4_hand(nf.quantize)
    check_nvfp4_blocks_along_k(nf.quantize)
    # all-zero tensor: S = 1, scales and codes 0
    q, s, S = nf.quantize(np.zeros((3, 64), np.float32))
    assert S == 1.0 and not s.any() and not q.any()
    # dequantized values stay within one E2M1 step (at most 2 units of s*S) of the input
    X = (rng(62).standard_normal((8, 128)) * np.exp(rng(63).uniform(-5, 5, (8, 1)))).astype(np.float32)
    q, s, S = nf.quantize(X)
    step = np.repeat(s.astype(np.float64) * S, 16, axis=1)
    assert np.all(np.abs(nf.dequantize(q, s, S) - X) <= 1.0 * step * 1.0001 + 1e-30)


def test_nvfp4_pin_catches_blocks_along_rows():
    from oracle import nvfp4 as nf

    def along_rows(X):  # blocks of 16 rows in a column instead of 16 elements of a row
        q, s, S = nf.quantize(np.ascontiguousarray(np.asarray(X, np.float32).T))
        return q.T, s.T, S

    with pytest.raises(Exception):
        check_nvfp4_blocks_along_k(along_rows)


def check_nvfp4_gemm_exact(gemm):
    # tiny case against exact rational arithmetic
    from oracle import nvfp4 as nf
    r = rng(64)
    A = (r.standard_normal((2, 32)) * 3).astype(np.float32)
    W = (r.standard_normal((3, 32)) * 0.2).astype(np.float32)
    bias = np.array([0.5, -1.25, 3.0])
    qa, sa, Sa = nf.quantize(A)
    qw, sw, Sw = nf.quantize(W)
    Y = gemm(qa, sa, Sa, qw, sw, Sw, bias)
    for m in range(2):
        for n in range(3):
            acc = Fraction(0)
            for k in range(32):
                acc += (Fraction(float(qa[m, k])) * Fraction(float(sa[m, k // 16]))
                        * Fraction(float(qw[n, k])) * Fraction(float(sw[n, k // 16])))
            want = acc * Fraction(float(Sa)) * Fraction(float(Sw)) + Fraction(bias[n])
            assert abs(Fraction(Y[m, n]) - want) <= abs(want) * Fraction(1, 2 ** 50)


def test_nvfp4_gemm_pins():
    from oracle import nvfp4 as nf
    check_nvfp4_gemm_exact(nf.gemm)


def test_nvfp4_gemm_pin_catches_missing_tensor_scale():
    from oracle import nvfp4 as nf

    def no_global(qa, sa, Sa, qw, sw, Sw, bias=None):
        return nf.gemm(qa, sa, 1.0, qw, sw, Sw, bias)

    with pytest.raises(AssertionError):
        check_nvfp4_gemm_exact(no_global)


def check_nvfp4_reciprocal_encoding(quantize):
    """The element encoding multiplies by the block's fp32 reciprocal, the convention of the
    INT8 quantizer reading (one IEEE division per block for inv, an fp32 product per element),
    and this block tells it apart from a per-element division. Row 1 holds 2688 = 6 * 448, so
    the tensor scale is S = 1; row 0's largest magnitude 5.625 gives the block scale
    5.625 / 6 = 0.9375 (an E4M3 value). Its other elements are 1.25, 2.5 and 5 times 0.9375:
    E2M1 midpoints exactly under division (ties to even: 1, 2, 4), but times fl32(1 / 0.9375)
    they land just above the midpoints (1.5, 3, 6). The expected codes are computed here with
    torch's fp32 arithmetic and a threshold count, not with the oracle's routines."""
    X = np.zeros((2, 16), np.float32)
    X[0, :4] = [5.625, 1.171875, 2.34375, 4.6875]
    X[1, 0] = 2688.0
    q, s, S = quantize(X)
    St = torch.tensor(2688.0, dtype=torch.float32) / torch.tensor(6.0 * 448.0, dtype=torch.float32)
    assert float(S) == float(St) == 1.0
    sb = (torch.tensor(5.625) / (6.0 * St)).to(torch.float8_e4m3fn).float()
    assert float(s[0, 0]) == float(sb) == 0.9375
    inv = torch.reciprocal(sb * St)  # fp32
    y = torch.from_numpy(X[0, :4]) * inv
    want = [_e2m1_by_thresholds(float(v)) for v in y]
    assert want == [6.0, 1.5, 3.0, 6.0]
    assert np.array_equal(q[0, :4], np.array(want, np.float32))


def test_nvfp4_encoding_is_multiplication_by_the_block_reciprocal():
    from oracle import nvfp4 as nf
    check_nvfp4_reciprocal_encoding(nf.quantize)


def test_nvfp4_reciprocal_pin_catches_per_element_division():
    from oracle import nvfp4 as nf
    bad_rows = planted(nf.quantize_rows, "v = (blocks * inv[..., None]).astype(np.float32)",
                       "v = (blocks / np.where(denom > 0, denom, np.float32(1))[..., None]).astype(np.float32)")

    def bad(X):
        S = nf.tensor_scale(X)
        q, s = bad_rows(X, S)
        return q, s, S

    with pytest.raises(AssertionError):
        check_nvfp4_reciprocal_encoding(bad)


def check_nvfp4_gemm_abs(gemm_abs):
    """gemm_abs = S_A S_W sum_k |q_A s_A| |q_W s_W|, the scale of the GEMM's fp32 accumulation
    error: exact rational arithmetic on a tiny mixed-sign case; equal to the GEMM itself for
    nonnegative operands; never below |Y|, and above it where signs mix."""
    from oracle import nvfp4 as nf
    r = rng(65)
    A = (r.standard_normal((2, 32)) * 3).astype(np.float32)
    W = (r.standard_normal((3, 32)) * 0.2).astype(np.float32)
    qa, sa, Sa = nf.quantize(A)
    qw, sw, Sw = nf.quantize(W)
    G = gemm_abs(qa, sa, qw, sw, Sa, Sw)
    for m in range(2):
        for n in range(3):
            acc = Fraction(0)
            for k in range(32):
                acc += (abs(Fraction(float(qa[m, k])) * Fraction(float(sa[m, k // 16])))
                        * abs(Fraction(float(qw[n, k])) * Fraction(float(sw[n, k // 16]))))
            want = acc * Fraction(float(Sa)) * Fraction(float(Sw))
            assert abs(Fraction(G[m, n]) - want) <= want * Fraction(1, 2 ** 50)
    Y = nf.gemm(qa, sa, Sa, qw, sw, Sw)
    assert np.all(G >= np.abs(Y)) and np.any(G > np.abs(Y) * 1.01)
    qp, sp, Sp = nf.quantize(np.abs(A))
    qv, sv, Sv = nf.quantize(np.abs(W))
    np.testing.assert_allclose(gemm_abs(qp, sp, qv, sv, Sp, Sv), nf.gemm(qp, sp, Sp, qv, sv, Sv), rtol=1e-15, atol=0)


def test_nvfp4_gemm_abs_pins():
    from oracle import nvfp4 as nf
    check_nvfp4_gemm_abs(nf.gemm_abs)


def test_nvfp4_gemm_abs_pin_catches_missing_absolute_value():
    from oracle import nvfp4 as nf
    bad = planted(nf.gemm_abs, "A = np.abs(dequantize(qa, sa, 1.0))", "A = dequantize(qa, sa, 1.0)")
    with pytest.raises(AssertionError):
        check_nvfp4_gemm_abs(bad)
