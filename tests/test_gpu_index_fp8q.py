"""The indexer with FP8 queries (q_dtype | LCCA_Q_FP8) over FP8 keys.

* Parity: the device logits equal the oracle's logits of the quantised query
  (orc_quantize_fp8_rows per row and head, dequantised exactly) within the
  fp32 bound used for the bf16 path.
* Tolerance against the unquantised (bf16) query: every logit within the
  quantisation bound sum_h w_h sum_d max(2^-4 |q_hd|, 2^(X_h - 10)) |K_gd|
  (plus the fp32 bound), and the top-k sets' overlap with the bf16 query's
  selection (recall) at least 0.95 on these N(0,1) inputs.
* lcca_decode_select with the flag equals the separate calls with it.
Shapes: the lp_512k indexer (64 heads x 128), 32 x 256, 128 x 64; one head
of one row is all zeros (X = -127)."""
import numpy as np
import pytest
import torch

import compare as C
import oracle as O
from long_context_compressed_append_amd import lcca, synth
from state import State, pool_rows
from gpu_state import GpuState, DEV
from test_gpu_decode_select import _separate, _fused, _ld, _state_tensors

pytestmark = pytest.mark.gpu

S = synth.CONFIGS
CASES = [
    synth.shrink(S["lp_512k"], "q8_lp", (8191, 5002, 6003, 3), (1, 1, 1, 1), k=512),
    synth.shrink(S["lp_512k"], "q8_i32x256", (4095, 3001), (1, 1), k=256, HI=32, dI=256),
    synth.shrink(S["lp_512k"], "q8_i128x64", (4095, 3001, 2047), (1, 1, 1), k=256, HI=128, dI=64),
]
Q8 = lcca.BF16 | lcca.Q_FP8


def _state(cfg):
    st = State(cfg)
    q = st.q_idx.reshape(len(st.row_seq), cfg.HI, cfg.dI)
    q[0, 3, :] = 0                                    # a zero head
    return st


def _quantised(st):
    """The oracle's FP8 query (dequantised, exact in fp32) and each head's X."""
    c = st.cfg
    nr = len(st.row_seq)
    qf = O.bf16_decode(st.q_idx).astype(np.float32).reshape(nr * c.HI, c.dI)
    codes, X = O.quantize_fp8_rows(qf)
    qd = (O.fp8_decode(codes) * 2.0 ** X[:, None].astype(np.float64)).astype(np.float32)
    return qd.reshape(nr, c.HI, c.dI), X.reshape(nr, c.HI)


def _keys(st, r):
    c = st.cfg
    n = (st.row_pos[r] + 1) // c.m
    return st.ik.rows(pool_rows(st.bt, c.m, st.row_seq[r], np.arange(n)))


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_fp8_query_logits_parity_and_tolerance(cfg):
    print("fp8-query indexer", cfg.name, flush=True)
    st = _state(cfg)
    st.oracle_compress_append()
    gs = GpuState(st)
    gs.q_dt = Q8
    lg = gs.index().cpu().numpy()
    nr = len(st.row_seq)
    qd, X = _quantised(st)
    rows = np.arange(nr)
    want = O.index_logits(st.row_seq, st.row_pos, cfg.m, st.bt, O.F32, qd, cfg.HI, cfg.dI, st.w_idx, 1.0,
                          st.ik.as_dict(), cfg.max_entries)
    full = st.oracle_index(rows)
    qb = O.bf16_decode(st.q_idx).astype(np.float64).reshape(nr, cfg.HI, cfg.dI)
    n_r = (st.row_pos + 1) // cfg.m
    bound = np.zeros_like(want)
    quant = np.zeros_like(want)
    for r in rows:
        K = np.abs(_keys(st, r))
        w = st.w_idx[r].astype(np.float64)
        bound[r, :n_r[r]] = (w[:, None] * (np.abs(qd[r]).astype(np.float64) @ K.T)).sum(0)
        dq = np.maximum(2.0 ** -4 * np.abs(qb[r]), 2.0 ** (X[r][:, None].astype(np.float64) - 10))
        quant[r, :n_r[r]] = (w[:, None] * (dq @ K.T)).sum(0)
    C.check_logits(lg, want, bound, n_r)
    # against the bf16 query: the quantisation bound (plus the fp32 bound)
    for r in rows:
        d = np.abs(lg[r, :n_r[r]].astype(np.float64) - full[r, :n_r[r]])
        assert np.all(d <= quant[r, :n_r[r]] + 2e-5 * bound[r, :n_r[r]] + 1e-30), r
    # selection overlap with the bf16 query's top-k
    got = O.topk(st.row_pos, cfg.m, lg.astype(np.float64), cfg.k)
    ref = O.topk(st.row_pos, cfg.m, full, cfg.k)
    rec = []
    for r in rows:
        a, b = set(got[r][got[r] >= 0]), set(ref[r][ref[r] >= 0])
        rec.append(len(a & b) / max(1, len(b)))
    print("fp8-query top-k recall per row", np.round(rec, 4), flush=True)
    assert min(rec) >= 0.95


@pytest.mark.parametrize("cfg", CASES[:1], ids=[CASES[0].name])
def test_decode_select_with_fp8_queries_equals_the_three_calls(cfg):
    print("decode_select fp8-query", cfg.name, flush=True)
    st = _state(cfg)
    ld = _ld(cfg)
    a, b = GpuState(st), GpuState(st)
    a.q_dt = b.q_dt = Q8
    lg_a, idx_a = _separate(a, ld)
    lg_b, idx_b = _fused(b, ld)
    torch.cuda.synchronize()
    for key, ta in _state_tensors(a).items():
        assert torch.equal(ta.view(torch.uint8), _state_tensors(b)[key].view(torch.uint8)), key
    pos = st.row_pos.astype(np.int64)
    n_r = (pos + 1) // cfg.m
    fresh = (pos + 1) % cfg.m == 0
    assert fresh.any()
    la, lb = lg_a.cpu().numpy(), lg_b.cpu().numpy()
    qd, _ = _quantised(st)
    ikh = a.ik.data.cpu().numpy()
    for r in range(len(pos)):
        stop = n_r[r] - 1 if fresh[r] else n_r[r]
        assert np.array_equal(la[r, :stop].view(np.uint32), lb[r, :stop].view(np.uint32)), r
        if fresh[r]:
            g = n_r[r] - 1
            prow = int(pool_rows(st.bt, cfg.m, st.row_seq[r], [g])[0])
            k = O.fp8_decode(ikh[prow * cfg.dI:(prow + 1) * cfg.dI]).astype(np.float64)
            q = qd[r].astype(np.float64)
            w = st.w_idx[r].astype(np.float64)
            exact = float((w * np.maximum(q @ k, 0.0)).sum())
            bnd = float((w * (np.abs(q) @ np.abs(k))).sum())
            assert abs(lb[r, g] - exact) <= 2e-5 * bnd, (r, lb[r, g], exact)
            assert abs(la[r, g] - lb[r, g]) <= 4e-5 * bnd
    assert torch.equal(idx_a, idx_b)
