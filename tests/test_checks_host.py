"""The test-side checks on the CPU: they accept the oracle's own results and reject planted
errors (so a GPU test that passes them shows something)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import prologue as po
from tests import sa_checks as chk


def _prologue_case(seed, mode):
    r = np.random.default_rng(seed)
    X = torch.from_numpy(r.standard_normal((1, 2, 1000, 128)).astype(np.float32) * 3).bfloat16().float().numpy()
    g = r.uniform(0.5, 1.5, (2, 128)).astype(np.float32)
    grid = (10, 10, 10)
    Y64, bound = po.qk_prologue64(X, g, 1e-6, grid)
    if mode == "bf16":  # the fp32 reading's values rounded to bf16 (RNE) by torch
        vals = torch.from_numpy(po.qk_prologue(X, g, 1e-6, grid)).bfloat16().double().numpy()
        return vals, Y64, bound
    quant = oracle.quantize_fp8_blocks if mode == "fp8" else oracle.quantize_int8_blocks
    codes, _ = quant(po.qk_prologue(X, g, 1e-6, grid), 128)
    return codes.astype(np.float64), Y64, bound


@pytest.mark.parametrize("mode", ["int8fp8", "fp8", "bf16"])
def test_codes_against_definition_accepts_the_fp32_reading(mode):
    codes, Y64, bound = _prologue_case(3, mode)
    exc, tot = chk.codes_against_definition(codes, Y64, bound, 128, mode)
    assert tot == codes.size and exc <= tot // 10000


@pytest.mark.parametrize("mode", ["int8fp8", "fp8", "bf16"])
def test_codes_against_definition_rejects_a_moved_code(mode):
    codes, Y64, bound = _prologue_case(4, mode)
    # move the code of the element farthest from any boundary: the largest in block 2
    i = 256 + int(np.argmax(np.abs(Y64[0, 1, 256:384, 7])))
    if mode == "bf16":  # one bf16 step down
        c = codes[0, 1, i, 7]
        codes[0, 1, i, 7] = c - np.sign(c) * np.exp2(np.floor(np.log2(abs(c))) - 7)
    else:
        codes[0, 1, i, 7] += -1.0 if mode == "int8fp8" else -0.5 * np.sign(codes[0, 1, i, 7])
    with pytest.raises(AssertionError):
        chk.codes_against_definition(codes, Y64, bound, 128, mode)


def _quantized_case(seed):
    r = np.random.default_rng(seed)
    Q = (r.standard_normal((1, 2, 300, 16)) * 2).astype(np.float32)
    K = (r.standard_normal((1, 2, 300, 16)) * 2).astype(np.float32)
    V = r.standard_normal((1, 2, 300, 16)).astype(np.float32)
    p = oracle.plan(Q, K, 64, 64, 0.4)
    Qh, sq = oracle.quantize_int8_blocks(Q, 64)
    Kh, sk = oracle.quantize_int8_blocks(K, 64)
    Vq, sv = oracle.quantize_fp8_blocks(V, 64)
    return (Qh, sq, Kh, sk, Vq, sv, p, 64, 64)


def test_bf16_rne64_is_round_to_nearest_even_on_8_bits():
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7: ties go to the even significand (1); 1 + 3 2^-8
    # is the midpoint of 1 + 2^-7 and 1 + 2^-6: up to the even one; just above a midpoint rounds up
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, -(1 + 2.0 ** -8), 3.0, 0.1])
    want = np.array([1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -1.0, 3.0, 0.10009765625])
    assert np.array_equal(chk.bf16_rne64(x), want)


def test_check_quantized_accepts_the_quantized_oracle_rounded_to_bf16():
    args = _quantized_case(5)
    got = oracle.bf16_rne(oracle.attend_quantized(*args))
    r = chk.check_quantized(got, *args)
    assert r["err"] < 5e-3 and r["bound_frac"] <= 1 and 0.8 < r["rms_ratio"] < 1.25


@pytest.mark.parametrize("planted", ["scale", "row_sum_of_fp32_p", "dropped_tile"])
def test_check_quantized_rejects_planted_errors(planted):
    args = _quantized_case(6)
    Qh, sq, Kh, sk, Vq, sv, p, bq, bk = args
    if planted == "scale":  # the V scale off by 1 %
        got = oracle.attend_quantized(*args) * 1.01
    elif planted == "row_sum_of_fp32_p":  # the first reading of the row sum
        from tests.test_oracle_pins import planted as plant
        from oracle import blocksparse as ob
        old = plant(ob.attend_quantized, "p8.sum(axis=1, dtype=np.float64) / 256.0", "p.sum(axis=1, dtype=np.float64)")
        got = old(*args)
    else:  # the last kept block of every row skipped
        got = oracle.attend_quantized(Qh, sq, Kh, sk, Vq, sv, p[..., :-1].copy(), bq, bk)
    with pytest.raises(AssertionError):
        chk.check_quantized(oracle.bf16_rne(got), *args)
