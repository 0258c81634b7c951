"""Degenerate rows on the device against the oracle: rows at the start of a
sequence (no visible entry, or fewer than k), top-k lists holding -1 and
out-of-range entries and repeats, in both the split (few rows) and the
one-workgroup-per-row (many rows) attention plans."""
import numpy as np
import pytest
import torch

import oracle as O
import compare as C
from long_context_compressed_append_amd import lcca, synth
from state import State, pool_rows, _scatter
from gpu_state import GpuState, dev_typed

pytestmark = pytest.mark.gpu

S = synth.CONFIGS
EDGE = {
    # one sequence from position 0: rows at positions 0 .. 299 (n = 0 .. 75, k = 64)
    "start_rows": synth.shrink(S["prefill_8k"], "edge_start", (0,), (300,), k=64, win_cap=512),
    # decode rows with n = 0, 1, 16, 75 (fewer than k = 64 but the last)
    "short_rows": synth.shrink(S["csa_64k"], "edge_short", (1, 6, 63, 300), (1, 1, 1, 1), k=64),
}


def _say(*a):
    print(*a, flush=True)


# Split plans of the split merge (dense rows, m = 128): each (row, 16-dim
# tile of the values) folds its key splits in chunks of 8 (at most 8 splits)
# or 16, and above 16 splits four waves share them, every fourth chunk each.
MERGE = {
    # 40 rows of 7 .. 312 entries (5 .. 14 tiles with the window): 5 splits of
    # 3 tiles, the short rows' last splits empty
    "merge_few_splits": (synth.shrink(S["hca_1m"], "merge_few", tuple(1000 * (i + 1) for i in range(40)),
                                      (1,) * 40), 2, 8),
    # a row of 3,200 entries (104 tiles, one split each: the first three
    # waves fold two chunks) and one of 100 (8 tiles: the other waves' splits
    # all empty)
    "merge_many_splits": (synth.shrink(S["hca_1m"], "merge_many", (409599, 12799), (1, 1)), 65, 256),
}


def _index_bound(st, rows):
    """sum_h w_h sum_d |q_hd k_d| for every visible entry of the given rows."""
    c = st.cfg
    out = np.zeros((len(rows), c.max_entries))
    q = st.q_idx.reshape(len(st.row_seq), c.HI, c.dI)
    qf = O.bf16_decode(q).astype(np.float64)
    for i, r in enumerate(rows):
        b, n = st.row_seq[r], (st.row_pos[r] + 1) // c.m
        K = st.ik.rows(pool_rows(st.bt, c.m, b, np.arange(n)))
        out[i, :n] = (st.w_idx[r][:, None] * (np.abs(qf[r]) @ np.abs(K).T)).sum(0)
    return out


@pytest.mark.parametrize("name", list(EDGE))
def test_rows_with_few_or_no_entries(name):
    cfg = EDGE[name]
    _say("edge rows", name)
    st = State(cfg)
    st.oracle_compress_append()
    gs = GpuState(st)
    lg = gs.index()
    idx = gs.topk(lg)
    out, lse = gs.attn(idx)
    torch.cuda.synchronize()
    nrows = len(st.row_seq)
    rows = np.arange(nrows)
    n_r = (st.row_pos + 1) // cfg.m
    assert (n_r == 0).any() and (n_r < cfg.k).any()
    lg_h, idx_h = lg.cpu().numpy(), idx.cpu().numpy()
    # logits of the visible entries, top-k on identical logits, attention on identical lists
    C.check_logits(lg_h, st.oracle_index(rows), _index_bound(st, rows), n_r)
    assert np.array_equal(idx_h, O.topk(st.row_pos, cfg.m, lg_h.astype(np.float64), cfg.k))
    assert (idx_h[n_r == 0] == -1).all()
    o_want, l_want = st.oracle_attn(idx_h, rows)
    C.check_attention(out.cpu().numpy(), o_want, "bf16")
    assert np.abs(lse.cpu().numpy() - l_want).max() <= 1e-3


def test_lists_with_invalid_and_repeated_entries():
    cfg = synth.shrink(S["csa_64k"], "edge_lists", (9999, 4101, 3003), (1, 1, 1), k=512)
    _say("top-k lists with -1, out-of-range and repeated entries")
    st = State(cfg)
    st.oracle_compress_append()
    gs = GpuState(st)
    g = np.random.default_rng(5)
    nrows = len(st.row_seq)
    n_r = (st.row_pos + 1) // cfg.m
    idx = np.empty((nrows, cfg.k), np.int32)
    for r in range(nrows):
        v = g.integers(0, n_r[r], cfg.k)
        kind = g.random(cfg.k)
        v[kind < 0.1] = -1                                  # padding
        v[(kind >= 0.1) & (kind < 0.15)] = n_r[r] + g.integers(0, 50)   # beyond the visible entries
        v[(kind >= 0.15) & (kind < 0.2)] = v[0]             # repeats of one entry
        idx[r] = v
    out, lse = gs.attn(dev_typed(idx))
    torch.cuda.synchronize()
    o_want, l_want = st.oracle_attn(idx, np.arange(nrows))
    C.check_attention(out.cpu().numpy(), o_want, "bf16")
    assert np.abs(lse.cpu().numpy() - l_want).max() <= 1e-3


def test_score_far_above_the_first_keys():
    """One selected entry whose score exceeds every other key's by about 150
    (log2 units), in the middle of the list: the online softmax must move its
    reference max and rescale what it has accumulated (a weight taken
    against the earlier max would overflow).  The output is then the value of
    that entry (the oracle's softmax is one-hot to fp64 precision)."""
    cfg = synth.shrink(S["csa_64k"], "edge_peak", (9999, 4101), (1, 1), k=512)
    _say("selected entry with a score far above the window's")
    st = State(cfg)
    st.oracle_compress_append()
    nrows = len(st.row_seq)
    n_r = (st.row_pos + 1) // cfg.m
    g = np.random.default_rng(11)
    idx = np.stack([np.sort(g.choice(n_r[r], cfg.k, replace=False)).astype(np.int32) for r in range(nrows)])
    q = st.q.reshape(nrows, cfg.H, cfg.D)
    big = int(idx[0, 300])
    q[0, :, 0] = O.bf16_encode(np.float32([60.0]))[0]
    prow = pool_rows(st.bt, cfg.m, st.row_seq[0], [big])
    x = st.kv.rows(prow).astype(np.float32)
    x[0, 0] = 60.0
    _scatter(st.kv, prow, x)
    gs = GpuState(st)
    out, lse = gs.attn(dev_typed(idx))
    torch.cuda.synchronize()
    o_want, l_want = st.oracle_attn(idx, np.arange(nrows))
    # the peak dominates row 0 (every head): its output is the entry's value
    assert np.abs(o_want[0] - x[0][None, : cfg.dv]).max() < 1e-6
    C.check_attention(out.cpu().numpy(), o_want, "bf16")
    assert np.abs(lse.cpu().numpy() - l_want).max() <= 1e-3


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", list(MERGE))
def test_split_merge_regimes(name, out_dtype):
    cfg, ns_lo, ns_hi = MERGE[name]
    _say("split merge", name, out_dtype)
    st = State(cfg)
    st.oracle_compress_append()
    gs = GpuState(st)
    nr = len(st.row_seq)
    # the plan's split count, from its workspace: fp32 partial values and an
    # (m, l) pair per (row, split, head)
    wsb = lcca.sparse_attn_workspace_size(gs.rows, cfg.m, cfg.H, cfg.D, cfg.dv, 0, False, cfg.window)
    ns = int(round(wsb / (nr * cfg.H * (4 * cfg.dv + 8))))
    assert ns_lo <= ns <= ns_hi, ns
    bf = out_dtype == "bf16"
    out, lse = gs.attn(None, out_dtype=lcca.BF16 if bf else lcca.F32)
    torch.cuda.synchronize()
    o_want, l_want = st.oracle_attn(None)
    got = out.float().cpu().numpy()
    C.check_attention(got, o_want, "bf16", out_bf16=bf)
    if not bf:
        # fp32 outputs: scores of exact bf16 operands summed in fp32, P as a
        # bf16 hi + lo pair (16 significant bits), fp32 accumulators and
        # merge; the values are N(0,1), so every output is within 1e-4 (a
        # split dropped or weighted wrongly moves it by ~1e-3 or more)
        assert np.abs(got - o_want).max() <= 1e-4
    assert np.abs(lse.cpu().numpy() - l_want).max() <= 1e-3
