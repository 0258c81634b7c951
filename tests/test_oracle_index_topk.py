"""Pins for the oracle's indexer logits and top-k selection.

Indexer: the same logits computed with numpy matrix products on keys read
back through a closed-form page address; linearity in the head weights;
ReLU sign property; the one-head case; 40-digit decimal brute force.
Top-k: numpy's stable lexicographic sort (a library routine); exhaustive
subset search on tiny inputs; k >= n and padding; signed-zero ties."""
import numpy as np
import pytest

import oracle as O
import bruteforce as BF


def _pool(rng, batch, nblk, m, dim, dtype, n_per_seq):
    E = 256 // m
    bt = rng.permutation(batch * nblk).astype(np.int32).reshape(batch, nblk)
    data, scale = O.alloc_rows(dtype, batch * nblk * E, dim, dtype == O.MXFP4)
    keys = []
    for b in range(batch):
        x = rng.standard_normal((n_per_seq, dim)).astype(np.float32)
        for g in range(n_per_seq):
            O.store_rows(dtype, data, scale, int(bt[b, g // E]) * E + g % E, x[g:g + 1])
        keys.append(O.load_rows(dtype, data, scale, 0, batch * nblk * E, dim)[
            [int(bt[b, g // E]) * E + g % E for g in range(n_per_seq)]])
    return bt, dict(dtype=dtype, data=data, scale=scale), keys


@pytest.mark.parametrize("dtype", [O.F32, O.BF16, O.FP8])
def test_index_matches_numpy_formula(dtype):
    rng = np.random.default_rng(50 + dtype)
    m, HI, dI, batch = 4, 6, 48, 3
    n_per = 300
    bt, ik, keys = _pool(rng, batch, 5, m, dI, dtype, n_per)
    pos = np.array([1199, 640, 3], np.int32)          # ragged, one row with no full entry
    seq = np.arange(batch, dtype=np.int32)
    q = rng.standard_normal((batch, HI, dI)).astype(np.float32)
    w = rng.random((batch, HI)).astype(np.float32)
    ld = 320
    got = O.index_logits(seq, pos, m, bt, O.F32, q, HI, dI, w, 0.5, ik, ld)
    for r in range(batch):
        n = (pos[r] + 1) // m
        K = keys[r][:n]
        want = 0.5 * (np.maximum(q[r].astype(np.float64) @ K.T, 0) * w[r][:, None].astype(np.float64)).sum(0)
        assert np.allclose(got[r, :n], want, rtol=1e-12, atol=1e-12)
        assert np.all(got[r, n:] == 0)          # nothing beyond the visible entries


def test_index_linear_in_weights_and_nonnegative():
    rng = np.random.default_rng(60)
    bt, ik, _ = _pool(rng, 1, 2, 4, 32, O.BF16, 128)
    q = rng.standard_normal((1, 4, 32)).astype(np.float32)
    w1 = rng.random((1, 4)).astype(np.float32); w2 = rng.random((1, 4)).astype(np.float32)
    args = (np.zeros(1, np.int32), np.array([511], np.int32), 4, bt, O.F32, q, 4, 32)
    l1 = O.index_logits(*args, w1, 1.0, ik, 128)
    l2 = O.index_logits(*args, w2, 1.0, ik, 128)
    l12 = O.index_logits(*args, (w1 + w2).astype(np.float32), 1.0, ik, 128)
    ws = (w1.astype(np.float64) + w2)
    assert np.allclose(l12, l1 + l2, rtol=1e-6 if not np.array_equal(ws.astype(np.float32), ws) else 1e-12)
    assert np.all(l1 >= 0)
    # sign of q flips which heads pass the ReLU: l(q) + l(-q) = sum_h w_h |q_h . k|
    ln = O.index_logits(np.zeros(1, np.int32), np.array([511], np.int32), 4, bt, O.F32, -q, 4, 32, w1, 1.0, ik, 128)
    keys = O.load_rows(O.BF16, ik["data"], None, 0, 2 * 64, 32)
    rows = [int(bt[0, g // 64]) * 64 + g % 64 for g in range(128)]
    absdot = (np.abs(q[0].astype(np.float64) @ keys[rows].T) * w1[0][:, None]).sum(0)
    assert np.allclose(l1[0] + ln[0], absdot, rtol=1e-12)


def test_index_one_head_unit_weight_is_relu_dot():
    rng = np.random.default_rng(61)
    bt, ik, keys = _pool(rng, 1, 1, 4, 16, O.F32, 64)
    q = rng.standard_normal((1, 1, 16)).astype(np.float32)
    got = O.index_logits(np.zeros(1, np.int32), np.array([255], np.int32), 4, bt, O.F32, q, 1, 16,
                         np.ones((1, 1), np.float32), 1.0, ik, 64)
    assert np.allclose(got[0], np.maximum(keys[0] @ q[0, 0].astype(np.float64), 0), rtol=1e-13, atol=1e-14)


def test_index_decimal_bruteforce():
    rng = np.random.default_rng(62)
    bt, ik, keys = _pool(rng, 1, 1, 4, 8, O.F32, 12)
    q = rng.standard_normal((1, 3, 8)).astype(np.float32)
    w = rng.random((1, 3)).astype(np.float32)
    got = O.index_logits(np.zeros(1, np.int32), np.array([47], np.int32), 4, bt, O.F32, q, 3, 8, w, 2.0, ik, 12)
    for g in range(12):
        assert abs(got[0, g] - float(BF.index_logit(q[0], w[0], keys[0][g], 2.0))) <= 1e-13 * (1 + abs(got[0, g]))


# ---------------------------------------------------------------------------
# top-k
# ---------------------------------------------------------------------------

def _lexsort_topk(l, n, k):
    g = np.arange(n)
    order = np.lexsort((g, -l[:n]))            # primary: -l ascending; secondary: index
    return np.sort(order[:min(k, n)])


def test_topk_matches_lexsort_with_many_ties():
    rng = np.random.default_rng(70)
    rows, ld, m, k = 40, 3000, 4, 257
    logits = rng.integers(0, 50, (rows, ld)).astype(np.float64)     # heavy ties
    logits[::3] = rng.standard_normal((len(range(0, rows, 3)), ld))
    pos = rng.integers(0, ld * m, rows).astype(np.int32)
    got = O.topk(pos, m, logits, k)
    for r in range(rows):
        n = (pos[r] + 1) // m
        want = _lexsort_topk(logits[r], n, k)
        assert np.array_equal(got[r, :len(want)], want)
        assert np.all(got[r, len(want):] == -1)


def test_topk_exhaustive_subsets_tiny():
    rng = np.random.default_rng(71)
    for trial in range(60):
        n = int(rng.integers(1, 13)); k = int(rng.integers(1, 5))
        vals = rng.integers(-3, 4, n).astype(np.float64) * 0.5
        got = O.topk(np.array([n * 4 - 1], np.int32), 4, vals[None, :], k)[0]
        want = BF.topk_subset(vals, k)
        assert list(got[:len(want)]) == want, (vals, k)
        assert np.all(got[len(want):] == -1)


def test_topk_k_at_least_n_and_signed_zero():
    got = O.topk(np.array([19], np.int32), 4, np.array([[3.0, 1.0, 2.0, 0.5, 9.0]]), 8)
    assert list(got[0]) == [0, 1, 2, 3, 4, -1, -1, -1]
    z = np.array([[0.0, -0.0, 0.0, -0.0, 1.0]])
    got = O.topk(np.array([19], np.int32), 4, z, 3)
    assert list(got[0]) == [0, 1, 4]          # -0.0 ties +0.0; smaller index first
