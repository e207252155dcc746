"""bench.py's host-side helpers on the CPU: the clock line of the driver's listing and the count
of valid (query, key) pairs behind the reported MFMA rate."""
import numpy as np

import bench


def test_current_sclk_is_the_marked_line():
    busy = "0: 500Mhz\n1: 1878Mhz *\n"
    idle = "S: 103Mhz *\n0: 500Mhz\n1: 2400Mhz\n"
    assert bench.current_sclk_mhz(busy) == 1878
    assert bench.current_sclk_mhz(idle) == 103
    assert bench.current_sclk_mhz("0: 500Mhz\n1: 2400Mhz\n") is None


def test_valid_pairs_counts_every_query_key_pair_inside_the_kept_tiles():
    # brute force over a small ragged case: L = 300, query blocks of 64, key blocks of 32
    rng = np.random.default_rng(1)
    L, bq, bk = 300, 64, 32
    nQ, nK, nk = -(-L // bq), -(-L // bk), 4
    plan = np.stack([np.sort(rng.choice(nK, nk, replace=False)) for _ in range(2 * 3 * nQ)]).reshape(2, 3, nQ, nk)
    want = 0
    for b in range(2):
        for h in range(3):
            for i in range(nQ):
                for j in plan[b, h, i]:
                    for qrow in range(i * bq, min(L, (i + 1) * bq)):
                        want += sum(1 for kcol in range(j * bk, (j + 1) * bk) if kcol < L)
    assert bench.valid_pairs(plan, L, bq, bk) == want
