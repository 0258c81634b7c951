"""Pins for the oracle's compression (softmax-weighted aggregation of m
tokens) and for its paged append, window ring and remainder ring.

Checked against: invariants of the definition (weights sum to one, m=1 is
the identity, a one-hot group returns its token, constant groups, convex
hull, permutation and logit-shift invariance), a 40-digit decimal brute
force, and a closed-form page address computed here independently."""
import numpy as np
import pytest

import oracle as O
import bruteforce as BF


def test_m1_is_identity():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((1, 64))
    C = O.group_compress(x, [rng.standard_normal()])
    assert np.array_equal(C, x[0])


def test_weights_sum_to_one():
    for m in (4, 128):
        rng = np.random.default_rng(m)
        a = rng.standard_normal(m) * 3
        C = O.group_compress(np.ones((m, 5)), a)
        assert np.all(np.abs(C - 1.0) < 1e-15)


def test_one_hot_group_returns_token():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((4, 32))
    for hot in range(4):
        a = np.zeros(4); a[hot] = 1000.0
        assert np.array_equal(O.group_compress(x, a), x[hot])


def test_constant_group_and_convex_hull():
    rng = np.random.default_rng(12)
    v = rng.standard_normal(16)
    C = O.group_compress(np.tile(v, (128, 1)), rng.standard_normal(128))
    assert np.allclose(C, v, rtol=1e-14, atol=1e-15)
    x = rng.standard_normal((128, 200))
    C = O.group_compress(x, rng.standard_normal(128) * 2)
    assert np.all(C <= x.max(0) + 1e-15) and np.all(C >= x.min(0) - 1e-15)


def test_permutation_and_shift_invariance():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((4, 40)); a = rng.standard_normal(4)
    C = O.group_compress(x, a)
    perm = rng.permutation(4)
    assert np.allclose(O.group_compress(x[perm], a[perm]), C, rtol=1e-14, atol=1e-15)
    assert np.allclose(O.group_compress(x, a + 37.5), C, rtol=1e-13, atol=1e-14)
    # not invariant to permuting x alone (the weights follow their tokens)
    assert not np.allclose(O.group_compress(x[perm], a), C) or np.array_equal(perm, np.arange(4))


@pytest.mark.parametrize("m,dim", [(4, 8), (128, 3), (2, 5)])
def test_group_compress_matches_decimal(m, dim):
    rng = np.random.default_rng(100 + m)
    x = rng.standard_normal((m, dim)); a = rng.standard_normal(m) * 2
    C = O.group_compress(x, a)
    want = np.array([float(v) for v in BF.compress(x, a)])
    assert np.allclose(C, want, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------
# compress_append on a small paged cache
# ---------------------------------------------------------------------------

def _mk(batch, m, D, dI, dt, ik_dt, win_dt, cap, nblk_per_seq, rng):
    E = 256 // m
    nb = batch * nblk_per_seq
    bt = rng.permutation(nb).astype(np.int32).reshape(batch, nblk_per_seq)
    kv = dict(zip(("data", "scale"), O.alloc_rows(dt, nb * E, D, dt == O.MXFP4)), dtype=dt)
    ik = dict(zip(("data", "scale"), O.alloc_rows(ik_dt, nb * E, dI, False)), dtype=ik_dt)
    wd, ws = O.alloc_rows(win_dt, batch * cap, D, win_dt == O.FP8)
    win = dict(dtype=win_dt, cap=cap, data=wd, scale=ws)
    rem = dict(kv=np.zeros(batch * m * D * 4, np.uint8), ik=np.zeros(batch * m * dI * 4, np.uint8),
               kv_logit=np.zeros(batch * m, np.float32), ik_logit=np.zeros(batch * m, np.float32))
    return bt, kv, ik, win, rem


def _entry_closed_form(store, bt, m, b, g, dim):
    """Independent address computation: physical block bt[b][g // (256/m)],
    slot g % (256/m), row = block * (256/m) + slot."""
    E = 256 // m
    row = int(bt[b, g // E]) * E + g % E
    return O.load_rows(store["dtype"], store["data"], store["scale"], row, 1, dim)[0]


def _run_chunks(chunks, toks, logits, itoks, ilogits, state, m, D, dI):
    bt, kv, ik, win, rem = state
    batch = len(toks)
    pos = [0] * batch
    for sizes in chunks:             # sizes: tokens per sequence in this call
        cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        sp = np.asarray(pos, np.int32)
        kt = np.concatenate([toks[b][pos[b]:pos[b] + sizes[b]] for b in range(batch)]).astype(np.float32)
        kl = np.concatenate([logits[b][pos[b]:pos[b] + sizes[b]] for b in range(batch)]).astype(np.float32)
        it = np.concatenate([itoks[b][pos[b]:pos[b] + sizes[b]] for b in range(batch)]).astype(np.float32)
        il = np.concatenate([ilogits[b][pos[b]:pos[b] + sizes[b]] for b in range(batch)]).astype(np.float32)
        O.compress_append(bt, cu, sp, O.F32, kt, kl, it, il, m, D, dI, kv, ik, win, rem)
        pos = [pos[b] + sizes[b] for b in range(batch)]


@pytest.mark.parametrize("m", [4, 128, 1])
def test_append_entries_window_and_remainder(m):
    rng = np.random.default_rng(20 + m)
    batch, D, dI, cap = 3, 64, 32, 160
    lens = [1000, 517, 258] if m != 128 else [700, 383, 129]
    nblk = -(-max(lens) // 256)
    st = _mk(batch, m, D, dI, O.F32, O.F32, O.F32, cap, nblk, rng)
    bt, kv, ik, win, rem = st
    toks = [rng.standard_normal((L, D)).astype(np.float32) for L in lens]
    itoks = [rng.standard_normal((L, dI)).astype(np.float32) for L in lens]
    lg = [rng.standard_normal(L).astype(np.float32) for L in lens]
    ilg = [rng.standard_normal(L).astype(np.float32) for L in lens]
    _run_chunks([lens], toks, lg, itoks, ilg, st, m, D, dI)
    for b, L in enumerate(lens):
        n = L // m
        for g in sorted({0, n // 2, n - 1} if n else set()):
            want = np.array([float(v) for v in BF.compress(toks[b][g * m:(g + 1) * m], lg[b][g * m:(g + 1) * m])],
                            np.float32)
            assert np.array_equal(_entry_closed_form(kv, bt, m, b, g, D).astype(np.float32), want)
            wi = np.array([float(v) for v in BF.compress(itoks[b][g * m:(g + 1) * m], ilg[b][g * m:(g + 1) * m])],
                          np.float32)
            assert np.array_equal(_entry_closed_form(ik, bt, m, b, g, dI).astype(np.float32), wi)
        # entries of incomplete groups are not written
        if L % m:
            assert np.all(_entry_closed_form(kv, bt, m, b, n, D) == 0)
        # window: slot t % cap holds token t for the last cap tokens
        for t in range(max(0, L - cap), L):
            row = O.load_rows(O.F32, win["data"], None, b * cap + t % cap, 1, D)[0]
            assert np.array_equal(row.astype(np.float32), toks[b][t])
        # remainder ring: the tail tokens at slot t % m
        rk = rem["kv"].view(np.float32).reshape(batch, m, D)
        for t in range((L // m) * m, L):
            assert np.array_equal(rk[b, t % m], toks[b][t])
            assert rem["kv_logit"].reshape(batch, m)[b, t % m] == lg[b][t]


@pytest.mark.parametrize("dt,ik_dt,win_dt", [(O.BF16, O.BF16, O.FP8), (O.MXFP4, O.FP8, O.FP8),
                                              (O.F32, O.F32, O.BF16)])
def test_chunking_invariance(dt, ik_dt, win_dt):
    m, D, dI, cap, batch = 4, 64, 32, 128, 2
    rng = np.random.default_rng(30)
    lens = [777, 530]
    toks = [rng.standard_normal((L, D)).astype(np.float32) for L in lens]
    itoks = [rng.standard_normal((L, dI)).astype(np.float32) for L in lens]
    lg = [rng.standard_normal(L).astype(np.float32) for L in lens]
    ilg = [rng.standard_normal(L).astype(np.float32) for L in lens]
    nblk = 4

    def run(chunks):
        st = _mk(batch, m, D, dI, dt, ik_dt, win_dt, cap, nblk, np.random.default_rng(31))
        _run_chunks(chunks, toks, lg, itoks, ilg, st, m, D, dI)
        return st

    one = run([lens])
    # random chunking, including empty chunks for one sequence
    sizes, left = [], list(lens)
    r2 = np.random.default_rng(32)
    while any(left):
        s = [int(min(l, r2.integers(0, 90))) for l in left]
        sizes.append(s); left = [l - x for l, x in zip(left, s)]
    many = run(sizes)
    ones = run([[1 if p < L else 0 for L in lens] for p in range(max(lens))])
    for other in (many, ones):
        for a, b in zip(one[1:4], other[1:4]):
            assert np.array_equal(a["data"], b["data"])
            if a["scale"] is not None:
                assert np.array_equal(a["scale"], b["scale"])
        for b_, L in enumerate(lens):
            for t in range((L // m) * m, L):
                s = b_ * m + t % m
                assert np.array_equal(one[4]["kv"].view(np.float32).reshape(-1, D)[s],
                                      other[4]["kv"].view(np.float32).reshape(-1, D)[s])


def test_bf16_storage_is_rounded_compression():
    """A bf16 pool entry is the RNE bf16 code of the fp32-rounded exact aggregate."""
    m, D, dI, cap = 4, 32, 32, 128
    rng = np.random.default_rng(40)
    st = _mk(1, m, D, dI, O.BF16, O.BF16, O.FP8, cap, 1, rng)
    x = rng.standard_normal((8, D)).astype(np.float32)
    a = rng.standard_normal(8).astype(np.float32)
    _run_chunks([[8]], [x], [a], [x[:, :dI]], [a], st, m, D, dI)
    kv = st[1]
    for g in range(2):
        exact = np.array([float(v) for v in BF.compress(x[g * m:(g + 1) * m], a[g * m:(g + 1) * m])], np.float32)
        got = _entry_closed_form(kv, st[0], m, 0, g, D)
        assert np.array_equal(got, O.bf16_decode(O.bf16_encode(exact)))
