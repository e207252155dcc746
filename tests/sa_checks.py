"""Test-side helpers: decode the library's workspace layouts, compare plans with the
near-tie rule, error norms. Independent of the HIP sources (the layouts are re-derived
here from their description in include/sparse_attn.h)."""
from __future__ import annotations

import numpy as np

import oracle


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ---------------------------------------------------------------- workspace layouts
def workspace_pieces(ws, lay, B, H, bq, bk, mode):
    """The bytes of every piece a prepare pass writes (the alignment gaps are never written)."""
    BH, nQ, nK = B * H, lay["nQ"], lay["nK"]
    if mode in ("int8fp8", "fp8"):
        sizes = {"q_off": BH * nQ * bq * 128, "k_off": BH * nK * bk * 128, "v_off": BH * nK * bk * 128,
                 "sq_off": BH * nQ * 4, "sk_off": BH * nK * 4, "sv_off": BH * nK * 4}
    else:
        # K and V^T tiles and the Q-source word (the Q region is written only with the prologue)
        sizes = {"k_off": BH * nK * bk * 128 * 2, "v_off": BH * nK * bk * 128 * 2, "sq_off": 4}
    return {k: ws[lay[k]: lay[k] + n] for k, n in sizes.items()}



def decode_q_int8(ws, lay, B, H, L, bq):
    n = B * H * lay["nQ"] * bq * 128
    q = ws[lay["q_off"]: lay["q_off"] + n].view(np.int8).reshape(B, H, lay["nQ"] * bq, 128)
    return q[:, :, :L], q[:, :, L:]


def _unswizzle_rows(tiles, chunk_bytes, key_fn):
    # tiles [..., R, W]: byte c*chunk + e of row r stored at ((c ^ key(r)) * chunk + e)
    R, W = tiles.shape[-2:]
    nch = W // chunk_bytes
    out = np.empty_like(tiles)
    for r in range(R):
        k = key_fn(r)
        for c in range(nch):
            p = c ^ k
            out[..., r, c * chunk_bytes:(c + 1) * chunk_bytes] = tiles[..., r, p * chunk_bytes:(p + 1) * chunk_bytes]
    return out


def decode_k(ws, lay, B, H, L, bk, esize=1):
    nsub = bk // 64
    n = B * H * lay["nK"] * bk * 128 * esize
    raw = ws[lay["k_off"]: lay["k_off"] + n].reshape(B, H, lay["nK"] * nsub, 64, 128 * esize)
    key = (lambda r: (r >> 1) & 7) if esize == 1 else (lambda r: r & 15)
    logical = _unswizzle_rows(raw, 16, key)
    logical = logical.reshape(B, H, lay["nK"] * bk, 128 * esize)
    return logical[:, :, :L], logical[:, :, L:]


def fp8_pos_to_key(pos):
    # row position 32g + 16kb + 4w + r holds key 32kb + 8w + 4g + r
    g, rest = divmod(pos, 32)
    kb, rest = divmod(rest, 16)
    w, r = divmod(rest, 4)
    return 32 * kb + 8 * w + 4 * g + r


def bf16_pos_to_key(pos):
    # row position 16(2kb + w//2) + 8g + 4(w%2) + r holds key 32kb + 8w + 4g + r
    kc, rest = divmod(pos, 16)
    kb, wh = divmod(kc, 2)
    g, rest = divmod(rest, 8)
    wl, r = divmod(rest, 4)
    w = 2 * wh + wl
    return 32 * kb + 8 * w + 4 * g + r


def decode_vt_fp8(ws, lay, B, H, L, bk):
    nsub = bk // 64
    n = B * H * lay["nK"] * bk * 128
    raw = ws[lay["v_off"]: lay["v_off"] + n].reshape(B, H, lay["nK"] * nsub, 128, 64)
    rows = _unswizzle_rows(raw, 16, lambda d: (d >> 2) & 3)  # [.., d, pos]
    keys = np.array([fp8_pos_to_key(p) for p in range(64)])
    v = np.empty(raw.shape[:-2] + (64, 128), np.uint8)
    v[..., keys, :] = np.swapaxes(rows, -1, -2)  # [.., pos, d] -> key order
    v = v.reshape(B, H, lay["nK"] * bk, 128)
    return v[:, :, :L], v[:, :, L:]


def decode_vt_bf16(ws, lay, B, H, L, bk):
    nsub = bk // 64
    n = B * H * lay["nK"] * bk * 128 * 2
    raw = ws[lay["v_off"]: lay["v_off"] + n].reshape(B, H, lay["nK"] * nsub, 128, 128)
    rows = _unswizzle_rows(raw, 16, lambda d: (d >> 1) & 7).view(np.uint16)  # [.., d, 64 pos]
    keys = np.array([bf16_pos_to_key(p) for p in range(64)])
    v = np.empty(rows.shape[:-2] + (64, 128), np.uint16)
    v[..., keys, :] = np.swapaxes(rows, -1, -2)
    v = v.reshape(B, H, lay["nK"] * bk, 128)
    return v[:, :, :L], v[:, :, L:]


def scales(ws, lay, B, H):
    nQ, nK = lay["nQ"], lay["nK"]
    sq = ws[lay["sq_off"]: lay["sq_off"] + 4 * B * H * nQ].view(np.float32).reshape(B, H, nQ)
    sk = ws[lay["sk_off"]: lay["sk_off"] + 4 * B * H * nK].view(np.float32).reshape(B, H, nK)
    sv = ws[lay["sv_off"]: lay["sv_off"] + 4 * B * H * nK].view(np.float32).reshape(B, H, nK)
    return sq, sk, sv


# ---------------------------------------------------------------- plans
def pooled_scores(qv, kv, bq, bk):
    """The oracle's pooled scores and, per (query block, key block), sum_d |Qbar_d Kbar_d| (the
    scale of the fp64 rounding error of a score computed in another order)."""
    qm, km = oracle.pool_block_means(qv, bq), oracle.pool_block_means(kv, bk)
    return oracle.block_scores(qm, km), np.abs(qm) @ np.swapaxes(np.abs(km), -1, -2)


def compare_plan(gpu_plan, scores, n_keep, mag=None, rel=1e-6, label=""):
    """Check a GPU plan against pooled scores (float64 [B,H,nQ,nK]) from the oracle.

    A row passes if it equals the oracle's top-n_keep set (lower index wins ties), or if
    every block in which the two sets differ scores within the near-tie band of the
    n_keep-th score s_k: |S - s_k| <= rel * |s_k| + f_S + f_k, where f is the rounding
    floor of a score summed in another order: 2^-44 sum_d |Qbar_d Kbar_d| (the fp64 sums of
    the block means and of the 128-term product each carry at most ~2^-45 of it); f = 0
    when mag (that sum, as pooled_scores returns it) is not given. Prints the excused rows
    and returns their number; raises AssertionError on any other difference."""
    gpu_plan = np.asarray(gpu_plan)
    B, H, nQ, nK = scores.shape
    assert gpu_plan.shape == (B, H, nQ, n_keep), gpu_plan.shape
    floor = np.zeros_like(scores) if mag is None else 2.0 ** -44 * mag
    excused = []
    idx = np.arange(nK)
    for b in range(B):
        for h in range(H):
            for i in range(nQ):
                row = gpu_plan[b, h, i]
                assert np.all(np.diff(row) > 0), f"row {(b, h, i)} not strictly ascending: {row}"
                assert row[0] >= 0 and row[-1] < nK, f"row {(b, h, i)} out of range"
                s = scores[b, h, i]
                order = np.lexsort((idx, -s))
                want = np.sort(order[:n_keep])
                if np.array_equal(row, want):
                    continue
                kth = order[n_keep - 1]
                sk = s[kth]
                diff = np.setxor1d(row, want)
                band = rel * abs(sk) + floor[b, h, i, diff] + floor[b, h, i, kth]
                if not np.all(np.abs(s[diff] - sk) <= band):
                    raise AssertionError(
                        f"plan row {(b, h, i)} differs outside the near-tie band: "
                        f"blocks {diff.tolist()} scores {s[diff].tolist()} k-th {sk}")
                excused.append(((b, h, i), diff.tolist(), float(np.abs(s[diff] - sk).max() / abs(sk))))
    for where, blocks, gap in excused:
        print(f"  {label}near-tie row {where}: blocks {blocks} within {gap:.1e} (relative) of the k-th score",
              flush=True)
    return len(excused)


# ---------------------------------------------------------------- quantized outputs
# The FP8 MFMA sums its 64 products per instruction to within 2^-11.8 of the largest one
# (tests/test_gpu_hw.py measures it), so an all-FP8 score carries an error of at most
# 2 * 2^-11.8 of its largest product, below 2^-10 of the sum of its |products|.
FP8_SCORE_REL_ERR = 2.0 ** -10


def check_quantized(got, Qh, sq, Kh, sk, Vq, sv, plan, bq, bk, rows=None, qk_fp8=False, sm=None,
                    rms_ratio_max=1.25, contract=5e-3):
    """Check quantized-path outputs two ways and return the figures.

    1. Against the tile-by-tile quantized oracle (Q2): rel-L2 <= contract (the bar for the
       quantized path).
    2. Against exact softmax attention over the dequantized operands, which no choice of
       tile order, reference max or operation sequence shapes: every element within
       oracle.quantized_error_bound (P's FP8 rounding, float32 arithmetic, bf16 output; plus
       the FP8 MFMA's score sums for all-FP8 Q/K), and, for INT8 scores, the RMS distance
       within rms_ratio_max of the size that bound function predicts from the rounding
       steps alone.
    got: float array [B, H, L, d] (NaN-free where rows are given)."""
    want = oracle.attend_quantized(Qh, sq, Kh, sk, Vq, sv, plan, bq, bk, sm=sm, rows=rows)
    exact, bound, rms = oracle.quantized_error_bound(
        Qh, sq, Kh, sk, Vq, sv, plan, bq, bk, sm=sm, rows=rows,
        score_rel_err=FP8_SCORE_REL_ERR if qk_fp8 else 0.0)
    sel = ~np.isnan(want)
    g = np.asarray(got, np.float64)[sel]
    err = rel_l2(g, want[sel])
    dev = np.abs(g - exact[sel])
    worst = float((dev / bound[sel]).max())
    ratio = float(np.linalg.norm(g - exact[sel]) / np.linalg.norm(rms[sel]))
    assert np.isfinite(g).all()
    assert err <= contract, f"rel-L2 {err:.3e} against the quantized oracle exceeds {contract}"
    assert worst <= 1.0, f"an element lies {worst:.3f} x the bound from exact attention"
    if not qk_fp8:
        assert ratio <= rms_ratio_max, f"RMS distance from exact attention {ratio:.3f} x the predicted"
    return {"err": err, "bound_frac": worst, "rms_ratio": ratio,
            "err_exact": rel_l2(g, exact[sel])}


def fmt(r):
    return (f"rel-L2 vs quantized oracle {r['err']:.2e}; vs exact attention {r['err_exact']:.2e}, "
            f"worst element {r['bound_frac']:.3f} of the bound, RMS {r['rms_ratio']:.3f} x predicted")


# ---------------------------------------------------------------- codes against fp64 definitions
def bf16_rne64(y):
    """float64 values rounded to bf16 (8 significant bits, nearest, ties to even), in one step
    from float64 (normal range)."""
    m, e = np.frexp(np.asarray(y, np.float64))  # y = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def codes_against_definition(gpu_vals, Y64, bound, b, mode, where=""):
    """Quantized codes of a prologue output (gpu_vals: the library's INT8 codes, E4M3 values or,
    for mode "bf16", bf16 values, [B, H, L, d]) against the codes the fp64 definition Y64 gives,
    under the same quantizer reading. An element may differ only where the fp32 operation sequence (values within
    `bound` of Y64) can reach the other side of a rounding boundary: its quantized value t64
    within delta of a boundary, delta bounding |t32 - t64| from the value's bound and the block
    maximum's. A whole FP8 block is excused when its maximum sits within its bound of a
    power-of-two scale boundary. Returns (excused elements, total)."""
    B, H, L, d = Y64.shape
    excused = 0
    for lo, hi in oracle.block_bounds(L, b):
        y = Y64[:, :, lo:hi]
        by = bound[:, :, lo:hi]
        g = np.asarray(gpu_vals[:, :, lo:hi], np.float64)
        amax = np.abs(y).max(axis=(2, 3), keepdims=True)
        bmax = by.max(axis=(2, 3), keepdims=True)
        zero = amax == 0
        amax = np.where(zero, 1.0, amax)
        if mode == "bf16":  # no block scale: each value rounded to bf16 on its own
            want = bf16_rne64(y)
            ex = np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -126)))
            step = np.exp2(ex - 7)
            frac = np.abs(np.abs(y) / step - np.floor(np.abs(y) / step) - 0.5) * step
            near = frac <= 2 * by
            bad = (g != want) & ~near
            assert not bad.any(), (f"{where}block [{lo},{hi}): {int(bad.sum())} values differ from the "
                                   f"fp64 definition's bf16 rounding away from any rounding boundary")
            excused += int(((g != want) & near).sum())
            continue
        if mode == "int8fp8":
            t = y * 127.0 / amax
            want = np.clip(np.rint(t), -127, 127)
            delta = 2 * (127.0 * by / amax + np.abs(t) * (bmax / amax + 2.0 ** -23))
            frac = np.abs(t - np.floor(t) - 0.5)  # distance to the nearest k + 1/2
            near = frac <= delta
        else:
            e = oracle.fp8_block_exponent(amax.astype(np.float32)).astype(np.float64)
            t = y * np.exp2(-e)
            want = oracle.e4m3_rne(np.clip(t, -448, 448).astype(np.float32)).astype(np.float64)
            scale_near = np.abs(amax - 448.0 * np.exp2(e)) <= 2 * bmax  # e itself could move
            # E4M3 rounding boundaries around t: midpoints of the grid step at |t|
            ex = np.maximum(np.floor(np.log2(np.maximum(np.abs(t), 2.0 ** -6))), -6)
            step = np.exp2(ex - 3)
            frac = np.abs(np.abs(t) / step - np.floor(np.abs(t) / step) - 0.5) * step
            delta = 2 * (by * np.exp2(-e) + np.abs(t) * 2.0 ** -23)
            near = (frac <= delta) | scale_near
        want = np.where(zero, 0.0, want)
        near = near & ~zero
        bad = (g != want) & ~near
        assert not bad.any(), (f"{where}block [{lo},{hi}): {int(bad.sum())} codes differ from the fp64 "
                               f"definition away from any rounding boundary")
        excused += int(((g != want) & near).sum())
    return excused, Y64.size
