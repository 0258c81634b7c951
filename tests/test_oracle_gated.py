"""Pins for the oracle's per-channel-gated compression (every channel of every
token has its own logit; the softmax over the group's m tokens is taken per
channel) and for its gated paged append.

Checked against: invariants of the definition (m=1 is the identity, each
channel's weights sum to one, per-channel shift invariance, a dominant logit
per channel returns that token's value in that channel), the special case of
channel-uniform logits, which is the per-token compression (pinned on its
own), a 40-digit decimal brute force per channel, the closed-form page
address, chunking invariance, and the remainder ring's per-channel logits."""
import numpy as np
import pytest

import oracle as O
import bruteforce as BF

from test_oracle_compress import _entry_closed_form


def test_m1_is_identity():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 33)); a = rng.standard_normal((1, 33)) * 5
    assert np.array_equal(O.group_compress_gated(x, a), x[0])


def test_each_channels_weights_sum_to_one():
    rng = np.random.default_rng(2)
    for m in (2, 4, 16, 128):
        a = rng.standard_normal((m, 40)) * 3
        C = O.group_compress_gated(np.ones((m, 40)), a)
        assert np.allclose(C, 1.0, rtol=0, atol=4e-16 * m)


def test_per_channel_shift_invariance():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 24)); a = rng.standard_normal((8, 24))
    shift = rng.standard_normal(24) * 50            # a different shift per channel
    C = O.group_compress_gated(x, a)
    assert np.allclose(O.group_compress_gated(x, a + shift[None, :]), C, rtol=1e-13, atol=1e-14)


def test_dominant_logit_per_channel_selects_that_token():
    rng = np.random.default_rng(4)
    m, dim = 8, 16
    x = rng.standard_normal((m, dim))
    a = rng.uniform(-1, 0, (m, dim))
    pick = rng.integers(0, m, dim)                  # a different winner in each channel
    a[pick, np.arange(dim)] = 80.0
    C = O.group_compress_gated(x, a)
    assert np.allclose(C, x[pick, np.arange(dim)], rtol=1e-15, atol=1e-300)


def test_channel_uniform_logits_are_the_per_token_compression():
    rng = np.random.default_rng(5)
    for m in (1, 4, 128):
        x = rng.standard_normal((m, 20)); a = rng.standard_normal(m) * 2
        g = O.group_compress_gated(x, np.repeat(a[:, None], 20, axis=1))
        assert np.array_equal(g, O.group_compress(x, a))


@pytest.mark.parametrize("m,dim", [(1, 3), (2, 5), (4, 7), (8, 4), (4, 4)])
def test_group_compress_gated_matches_decimal(m, dim):
    rng = np.random.default_rng(200 + m)
    x = rng.standard_normal((m, dim)); a = rng.standard_normal((m, dim)) * 2
    C = O.group_compress_gated(x, a)
    # each channel on its own: the per-token definition over that channel's logits
    want = np.array([float(BF.compress([[x[i, d]] for i in range(m)], a[:, d])[0]) for d in range(dim)])
    assert np.allclose(C, want, rtol=1e-14, atol=1e-15)
    # a transposed logit matrix (a[d][i]) gives another answer
    if m == dim:
        assert not np.allclose(O.group_compress_gated(x, a.T.copy()), want)


# ---------------------------------------------------------------------------
# gated compress_append on a small paged cache
# ---------------------------------------------------------------------------

def _mk(batch, m, D, dI, dt, ik_dt, win_dt, cap, nblk, rng):
    E = 256 // m
    nb = batch * nblk
    bt = rng.permutation(nb).astype(np.int32).reshape(batch, nblk)
    kv = dict(zip(("data", "scale"), O.alloc_rows(dt, nb * E, D, dt == O.MXFP4)), dtype=dt)
    ik = dict(zip(("data", "scale"), O.alloc_rows(ik_dt, nb * E, dI, False)), dtype=ik_dt)
    wd, ws = O.alloc_rows(win_dt, batch * cap, D, win_dt == O.FP8)
    win = dict(dtype=win_dt, cap=cap, data=wd, scale=ws)
    rem = dict(kv=np.zeros(batch * m * D * 4, np.uint8), ik=np.zeros(batch * m * dI * 4, np.uint8),
               kv_logit=np.zeros(batch * m * D, np.float32), ik_logit=np.zeros(batch * m * dI, np.float32))
    return bt, kv, ik, win, rem


def _run_chunks(chunks, toks, lg, itoks, ilg, state, m, D, dI):
    """Append per-sequence chunks (sizes per call) with the gated oracle."""
    bt, kv, ik, win, rem = state
    batch = len(toks)
    pos = [0] * batch
    for sizes in chunks:
        cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        sp = np.asarray(pos, np.int32)
        cat = lambda arrs: np.concatenate([arrs[b][pos[b]:pos[b] + sizes[b]] for b in range(batch)]).astype(np.float32)
        O.compress_append(bt, cu, sp, O.F32, cat(toks), cat(lg), cat(itoks), cat(ilg), m, D, dI, kv, ik, win, rem,
                          gated=True)
        pos = [pos[b] + sizes[b] for b in range(batch)]


def _data(m, D, dI, lens, seed):
    rng = np.random.default_rng(seed)
    toks = [rng.standard_normal((L, D)).astype(np.float32) for L in lens]
    itoks = [rng.standard_normal((L, dI)).astype(np.float32) for L in lens]
    lg = [rng.standard_normal((L, D)).astype(np.float32) for L in lens]
    ilg = [rng.standard_normal((L, dI)).astype(np.float32) for L in lens]
    return toks, itoks, lg, ilg


@pytest.mark.parametrize("m", [4, 16, 1])
def test_gated_append_entries_and_remainder(m):
    batch, D, dI, cap = 2, 32, 16, 64
    lens = [301, 158]
    toks, itoks, lg, ilg = _data(m, D, dI, lens, 50 + m)
    st = _mk(batch, m, D, dI, O.F32, O.F32, O.F32, cap, 2, np.random.default_rng(51))
    _run_chunks([[120, 40], [181, 118]], toks, lg, itoks, ilg, st, m, D, dI)
    bt, kv, ik, win, rem = st
    for b, L in enumerate(lens):
        n = L // m
        for g in sorted({0, n // 2, n - 1}):
            sl = slice(g * m, (g + 1) * m)
            want = np.array([float(BF.compress([[v] for v in toks[b][sl, d]], lg[b][sl, d])[0]) for d in range(D)],
                            np.float32)
            assert np.array_equal(_entry_closed_form(kv, bt, m, b, g, D).astype(np.float32), want)
            wi = np.array([float(BF.compress([[v] for v in itoks[b][sl, d]], ilg[b][sl, d])[0]) for d in range(dI)],
                          np.float32)
            assert np.array_equal(_entry_closed_form(ik, bt, m, b, g, dI).astype(np.float32), wi)
        # the remainder ring holds the tail tokens and their per-channel logits
        for t in range((L // m) * m, L):
            s = b * m + t % m
            assert np.array_equal(rem["kv"].view(np.float32).reshape(-1, D)[s], toks[b][t])
            assert np.array_equal(rem["kv_logit"].reshape(-1, D)[s], lg[b][t])
            assert np.array_equal(rem["ik_logit"].reshape(-1, dI)[s], ilg[b][t])
        for t in range(max(0, L - cap), L):
            assert np.array_equal(O.load_rows(O.F32, win["data"], None, b * cap + t % cap, 1, D)[0].astype(np.float32),
                                  toks[b][t])


@pytest.mark.parametrize("dt,ik_dt,win_dt", [(O.BF16, O.BF16, O.FP8), (O.MXFP4, O.FP8, O.FP8)])
def test_gated_chunking_invariance(dt, ik_dt, win_dt):
    m, D, dI, cap, batch = 4, 64, 32, 128, 2
    lens = [377, 230]
    toks, itoks, lg, ilg = _data(m, D, dI, lens, 60)

    def run(chunks):
        st = _mk(batch, m, D, dI, dt, ik_dt, win_dt, cap, 2, np.random.default_rng(61))
        _run_chunks(chunks, toks, lg, itoks, ilg, st, m, D, dI)
        return st

    one = run([lens])
    sizes, left, r2 = [], list(lens), np.random.default_rng(62)
    while any(left):
        s = [int(min(l, r2.integers(0, 70))) for l in left]
        sizes.append(s); left = [l - x for l, x in zip(left, s)]
    many = run(sizes)
    for a, b in zip(one[1:4], many[1:4]):
        assert np.array_equal(a["data"], b["data"])
        if a["scale"] is not None:
            assert np.array_equal(a["scale"], b["scale"])


def test_gated_with_uniform_logits_is_the_per_token_append():
    m, D, dI, cap, batch = 4, 64, 32, 96, 2
    lens = [333, 97]
    toks, itoks, lg, ilg = _data(m, D, dI, lens, 70)
    lg1 = [a[:, 0].copy() for a in lg]
    ilg1 = [a[:, 0].copy() for a in ilg]
    lgu = [np.repeat(a[:, None], D, 1) for a in lg1]
    ilgu = [np.repeat(a[:, None], dI, 1) for a in ilg1]
    gated = _mk(batch, m, D, dI, O.BF16, O.FP8, O.FP8, cap, 2, np.random.default_rng(71))
    _run_chunks([[200, 50], [133, 47]], toks, lgu, itoks, ilgu, gated, m, D, dI)
    plain = _mk(batch, m, D, dI, O.BF16, O.FP8, O.FP8, cap, 2, np.random.default_rng(71))
    plain[4]["kv_logit"] = np.zeros(batch * m, np.float32)
    plain[4]["ik_logit"] = np.zeros(batch * m, np.float32)
    bt, kv, ik, win, rem = plain
    pos = [0, 0]
    for sizes in ([200, 50], [133, 47]):
        cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        cat = lambda arrs: np.concatenate([arrs[b][pos[b]:pos[b] + sizes[b]] for b in range(batch)]).astype(np.float32)
        O.compress_append(bt, cu, np.asarray(pos, np.int32), O.F32, cat(toks), cat(lg1), cat(itoks), cat(ilg1), m, D,
                          dI, kv, ik, win, rem)
        pos = [pos[b] + sizes[b] for b in range(batch)]
    for a, b in zip(gated[1:4], plain[1:4]):
        assert np.array_equal(a["data"], b["data"])
        if a["scale"] is not None:
            assert np.array_equal(a["scale"], b["scale"])
    assert np.array_equal(gated[4]["kv"], plain[4]["kv"])
