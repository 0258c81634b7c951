"""The window ring's capacity rule (include/lcca.h, window ring): rows attended
inside an appended chunk of n tokens need capacity >= window + n - 1.

Shown on the oracle: a chunk of 24 tokens appended from position 0 with a
window of 16, dense attention over the visible entries plus the window.  With
capacity window + n - 1 every row's output equals that of a ring large enough
to hold every position; with capacity = window, the chunk's later tokens
overwrite slots that its early rows still read, so those rows' outputs change,
while rows whose window slots were not overwritten (the last rows) stay equal.
"""
import numpy as np

import oracle as O

M, D, H, W, N = 4, 128, 8, 16, 24


def _run(cap):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([0x1CCA, 99, 1])))
    x = rng.standard_normal((N, D), dtype=np.float32)
    a = rng.standard_normal(N, dtype=np.float32)
    q = rng.standard_normal((N, H, D), dtype=np.float32)
    bt = np.zeros((1, 1), np.int32)
    kv = {"dtype": O.F32, "data": np.zeros(64 * D * 4, np.uint8), "scale": None}
    win = {"dtype": O.F32, "cap": cap, "data": np.zeros(cap * D * 4, np.uint8), "scale": None}
    rem = {"kv": np.zeros(M * D * 4, np.uint8), "ik": None, "kv_logit": np.zeros(M, np.float32), "ik_logit": None}
    O.compress_append(bt, np.array([0, N], np.int32), np.array([0], np.int32), O.F32, x, a, None, None, M, D, 0,
                      kv, None, win, rem)
    pos = np.arange(N, dtype=np.int32)
    out, _ = O.sparse_attn(np.zeros(N, np.int32), pos, M, bt, O.F32, q, H, D, D, 1 / np.sqrt(D), kv, None, 0, win, W)
    return out


def test_capacity_rule_for_rows_inside_a_chunk():
    ref = _run(64)                              # every position keeps its own slot
    ok = _run(W + N - 1)
    assert np.array_equal(ok, ref)
    small = _run(W)
    differs = [p for p in range(N) if not np.array_equal(small[p], ref[p])]
    # only the chunk's last `cap` tokens are written: tokens W .. N-1 land in
    # the slots of positions 0 .. N-W-1 (tokens below N - W are not written at
    # all), so every row whose window reaches a position below N - W reads a
    # wrong token: rows p with p - W + 1 <= N - W - 1, i.e. all but the last
    assert differs == list(range(N - 1)), differs
