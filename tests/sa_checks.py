"""Test-side helpers: decode the library's workspace layouts, compare plans with the
near-tie rule, error norms. Independent of the HIP sources (the layouts are re-derived
here from their description in include/sparse_attn.h)."""
from __future__ import annotations

import numpy as np


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
        sizes = {"k_off": BH * nK * bk * 128 * 2, "v_off": BH * nK * bk * 128 * 2}
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
    logical = _unswizzle_rows(raw, 16, lambda r: r & 7)
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
    rows = _unswizzle_rows(raw, 16, lambda d: (d >> 1) & 3)  # [.., d, pos]
    keys = np.array([fp8_pos_to_key(p) for p in range(64)])
    v = np.empty(raw.shape[:-2] + (64, 128), np.uint8)
    v[..., keys, :] = np.swapaxes(rows, -1, -2)  # [.., pos, d] -> key order
    v = v.reshape(B, H, lay["nK"] * bk, 128)
    return v[:, :, :L], v[:, :, L:]


def decode_vt_bf16(ws, lay, B, H, L, bk):
    nsub = bk // 64
    n = B * H * lay["nK"] * bk * 128 * 2
    raw = ws[lay["v_off"]: lay["v_off"] + n].reshape(B, H, lay["nK"] * nsub, 128, 128)
    rows = _unswizzle_rows(raw, 16, lambda d: d & 7).view(np.uint16)  # [.., d, 64 pos]
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
def compare_plan(gpu_plan, scores, n_keep, rel=1e-6):
    """Check a GPU plan against pooled scores (float64 [B,H,nQ,nK]) from the oracle.

    A row passes if it equals the oracle's top-n_keep set (lower index wins ties), or if
    every block in which the two sets differ scores within the near-tie band of the
    n_keep-th score: |S - s_k| <= max(rel*|s_k|, rel*max_j|S_j|). Returns the number of
    rows excused by the band; raises AssertionError on any other difference."""
    gpu_plan = np.asarray(gpu_plan)
    B, H, nQ, nK = scores.shape
    assert gpu_plan.shape == (B, H, nQ, n_keep), gpu_plan.shape
    excused = 0
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
                sk = s[order[n_keep - 1]]
                band = max(rel * abs(sk), rel * np.abs(s).max())
                diff = np.setxor1d(row, want)
                if not np.all(np.abs(s[diff] - sk) <= band):
                    raise AssertionError(
                        f"plan row {(b, h, i)} differs outside the near-tie band: "
                        f"blocks {diff.tolist()} scores {s[diff].tolist()} k-th {sk}")
                excused += 1
    return excused
