"""Pins for the oracle's sparse attention over selected entries + window.

Closed cases: with top-k covering every visible entry the result is plain
dense softmax attention over [entries; window tokens] (checked with torch's
scaled_dot_product_attention in fp64, a library routine); with m=1, k >= T
and a window covering the whole context every token appears twice, which
leaves dense attention over the T tokens unchanged.  Special cases: a single
key returns its value, sm_scale = 0 averages the values, an empty selection
attends to the window only.  Tiny inputs against a 40-digit decimal brute
force, and the end-to-end tiny workload through all four stages."""
import numpy as np
import pytest
import torch

import oracle as O
import bruteforce as BF
from long_context_compressed_append_amd import synth
from state import State


def _sdpa(q, K, d_v, scale):
    """q [H][D], K [n][D] float64 -> (o [H][d_v], lse [H]) via torch."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, None]          # [1,1,H,D]
    qt = qt.transpose(1, 2)                                               # [1,H,1,D]
    kt = torch.from_numpy(np.asarray(K, np.float64))[None, None].expand(1, qt.shape[1], -1, -1)
    vt = kt[..., :d_v]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=float(scale))
    s = (qt @ kt.transpose(-1, -2)) * scale
    return o[0, :, 0].numpy(), torch.logsumexp(s, -1)[0, :, 0].numpy()


def _small_cache(rng, m, D, T, cap, dtype=O.F32, win_dtype=O.F32):
    """One sequence of T tokens compressed through the oracle itself."""
    E = 256 // m
    nblk = -(-T // 256)
    bt = rng.permutation(nblk).astype(np.int32)[None]
    kv = dict(zip(("data", "scale"), O.alloc_rows(dtype, nblk * E, D, dtype == O.MXFP4)), dtype=dtype)
    wd, ws = O.alloc_rows(win_dtype, cap, D, win_dtype == O.FP8)
    win = dict(dtype=win_dtype, cap=cap, data=wd, scale=ws)
    rem = dict(kv=np.zeros(m * D * 4, np.uint8), ik=None, kv_logit=np.zeros(m, np.float32), ik_logit=None)
    x = rng.standard_normal((T, D)).astype(np.float32)
    a = rng.standard_normal(T).astype(np.float32)
    O.compress_append(bt, np.array([0, T], np.int32), np.zeros(1, np.int32), O.F32, x, a, None, None,
                      m, D, 0, kv, None, win, rem)
    return bt, kv, win, x


def _entries(kv, bt, m, n, D):
    E = 256 // m
    rows = [int(bt[0, g // E]) * E + g % E for g in range(n)]
    return O.load_rows(kv["dtype"], kv["data"], kv["scale"], 0, bt.size * E, D)[rows]


def _window(win, p, w, D):
    cap = win["cap"]
    ts = range(max(0, p - w + 1), p + 1)
    return np.stack([O.load_rows(win["dtype"], win["data"], win["scale"], t % cap, 1, D)[0] for t in ts])


@pytest.mark.parametrize("m,T,p,w,dtype,win_dtype", [
    (4, 1000, 999, 128, O.F32, O.F32), (4, 700, 301, 128, O.BF16, O.FP8), (128, 1300, 1299, 128, O.BF16, O.FP8),
    (4, 90, 40, 128, O.MXFP4, O.FP8)])
def test_topk_covering_all_is_dense_attention(m, T, p, w, dtype, win_dtype):
    rng = np.random.default_rng(80 + m + T)
    D, H, d_v, cap = 64, 5, 48, 1024
    bt, kv, win, _ = _small_cache(rng, m, D, T, cap, dtype, win_dtype)
    n = (p + 1) // m
    q = rng.standard_normal((1, H, D)).astype(np.float32)
    k = n + 7
    idx = np.full((1, k), -1, np.int32); idx[0, :n] = rng.permutation(n)       # any order
    out, lse = O.sparse_attn(np.zeros(1, np.int32), np.array([p], np.int32), m, bt, O.F32, q, H, D, d_v, 0.3,
                             kv, idx, k, win, w)
    outd, lsed = O.sparse_attn(np.zeros(1, np.int32), np.array([p], np.int32), m, bt, O.F32, q, H, D, d_v, 0.3,
                               kv, None, 0, win, w)
    K = np.concatenate([_entries(kv, bt, m, n, D), _window(win, p, w, D)])
    o_ref, l_ref = _sdpa(q[0], K, d_v, 0.3)
    assert np.allclose(out[0], o_ref, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse[0], l_ref, rtol=1e-13, atol=1e-13)
    assert np.allclose(outd, out, rtol=1e-13, atol=1e-14)          # dense mode == full selection


def test_m1_full_window_full_topk_is_dense_over_tokens():
    rng = np.random.default_rng(90)
    T, D, H = 200, 32, 3
    bt, kv, win, x = _small_cache(rng, 1, D, T, 256)
    q = rng.standard_normal((1, H, D)).astype(np.float32)
    idx = np.arange(T, dtype=np.int32)[None]
    out, lse = O.sparse_attn(np.zeros(1, np.int32), np.array([T - 1], np.int32), 1, bt, O.F32, q, H, D, D, 0.2,
                             kv, idx, T, win, T)
    o_ref, l_ref = _sdpa(q[0], x.astype(np.float64), D, 0.2)
    assert np.allclose(out[0], o_ref, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse[0], l_ref + np.log(2.0), rtol=1e-13)    # every token counted twice


def test_single_key_zero_scale_and_window_only():
    rng = np.random.default_rng(91)
    D, H = 32, 2
    bt, kv, win, x = _small_cache(rng, 4, D, 300, 512)
    q = rng.standard_normal((1, H, D)).astype(np.float32)
    z = np.zeros(1, np.int32)
    # position 0: no complete entry, window holds token 0 only -> o = v_0
    out, lse = O.sparse_attn(z, np.array([0], np.int32), 4, bt, O.F32, q, H, D, D, 1.0, kv, None, 0, win, 128)
    assert np.array_equal(out[0], np.tile(x[0].astype(np.float64), (H, 1)))
    # sm_scale = 0: the mean of the values
    idx = np.array([[5, 2, 9]], np.int32)
    out, _ = O.sparse_attn(z, np.array([299], np.int32), 4, bt, O.F32, q, H, D, D, 0.0, kv, idx, 3, win, 128)
    K = np.concatenate([_entries(kv, bt, 4, 74, D)[[5, 2, 9]], _window(win, 299, 128, D)])
    assert np.allclose(out[0], np.tile(K.mean(0), (H, 1)), rtol=1e-13, atol=1e-14)
    # entries the row cannot see yet (g >= n = (p+1)/m) are skipped like -1:
    # position 199 sees entries 0..49 only
    idx_bad = np.array([[5, 60, 2, 49, 50, 73, 9]], np.int32)
    idx_ok = np.array([[5, 2, 49, 9]], np.int32)
    out_b, lse_b = O.sparse_attn(z, np.array([199], np.int32), 4, bt, O.F32, q, H, D, D, 0.3, kv, idx_bad, 7, win, 128)
    out_o, lse_o = O.sparse_attn(z, np.array([199], np.int32), 4, bt, O.F32, q, H, D, D, 0.3, kv, idx_ok, 4, win, 128)
    assert np.array_equal(out_b, out_o) and np.array_equal(lse_b, lse_o)
    # empty selection (-1 only): the window alone
    idx = np.full((1, 4), -1, np.int32)
    out, _ = O.sparse_attn(z, np.array([299], np.int32), 4, bt, O.F32, q, H, D, D, 0.5, kv, idx, 4, win, 128)
    o_ref, _ = _sdpa(q[0], _window(win, 299, 128, D), D, 0.5)
    assert np.allclose(out[0], o_ref, rtol=1e-12, atol=1e-13)


def test_attention_decimal_bruteforce():
    rng = np.random.default_rng(92)
    D, H, d_v = 8, 2, 6
    bt, kv, win, _ = _small_cache(rng, 4, D, 40, 64)
    q = rng.standard_normal((1, H, D)).astype(np.float32)
    idx = np.array([[7, 1, 3]], np.int32)
    out, lse = O.sparse_attn(np.zeros(1, np.int32), np.array([37], np.int32), 4, bt, O.F32, q, H, D, d_v, 0.7,
                             kv, idx, 3, win, 5)
    K = np.concatenate([_entries(kv, bt, 4, 9, D)[[7, 1, 3]], _window(win, 37, 5, D)])
    o_bf, l_bf = BF.attention(q[0], K, d_v, 0.7)
    assert np.allclose(out[0], np.array([[float(v) for v in r] for r in o_bf]), rtol=1e-13, atol=1e-14)
    assert np.allclose(lse[0], [float(v) for v in l_bf], rtol=1e-14)


def test_tiny_workload_end_to_end_decimal():
    """The fp32 tiny workload through all four oracle stages, every stage
    re-derived with the decimal brute force from the raw seeded draws."""
    cfg = synth.CONFIGS["tiny"]
    st = State(cfg)
    st.oracle_compress_append()
    x, xi, a, ai = synth.new_tokens(cfg, 0)
    m, n = cfg.m, 256
    # compressed entries and indexer keys straight from the tokens
    Kc = np.array([[float(v) for v in BF.compress(x[g * m:(g + 1) * m], a[g * m:(g + 1) * m])]
                   for g in range(n)], np.float32).astype(np.float64)
    Ki = np.array([[float(v) for v in BF.compress(xi[g * m:(g + 1) * m], ai[g * m:(g + 1) * m])]
                   for g in range(n)], np.float32).astype(np.float64)
    logits = st.oracle_index()
    q, qi, w = synth.queries(cfg, 0, 1)
    want_l = np.array([float(BF.index_logit(qi[0], w[0], Ki[g])) for g in range(n)])
    assert np.allclose(logits[0, :n], want_l, rtol=1e-12, atol=1e-12)
    idx = st.oracle_topk(logits)
    assert list(idx[0]) == sorted(np.argsort(-want_l, kind="stable")[:cfg.k])
    out, lse = st.oracle_attn(idx)
    K = np.concatenate([Kc[idx[0]], x[-128:].astype(np.float64)])
    o_bf, l_bf = BF.attention(q[0], K, cfg.D, cfg.scale)
    assert np.allclose(out[0], np.array([[float(v) for v in r] for r in o_bf]), rtol=1e-12, atol=1e-13)
    assert np.allclose(lse[0], [float(v) for v in l_bf], rtol=1e-13)
