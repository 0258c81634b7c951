"""lcca_decode_select (compress_append + index_logits + topk_select of a
decode step with one launch fewer) against the three separate calls on identical
device copies of the same state: pools, window and remainder rings and the
logits of every entry already in the pool bit for bit; the logit of the entry
a row's own token completes (formed and scored inside the indexer launch)
within the fp32 bound of the oracle's tolerance; identical top-k lists; and
the top-k lists of the separate calls equal the oracle's selection on the
same logits."""
import numpy as np
import pytest
import torch

import oracle as O
from long_context_compressed_append_amd import lcca, synth
from state import State, pool_rows
from gpu_state import GpuState, DEV

pytestmark = pytest.mark.gpu

S = synth.CONFIGS
CASES = {
    # positions 9999 and 3003 complete a group (m = 4), 4101 does not
    "csa_mixed": synth.shrink(S["csa_64k"], "ds_mixed", (9999, 4101, 3003), (1, 1, 1), k=512),
    # every row completes a group; the last one its first (one visible entry)
    "csa_all_fresh": synth.shrink(S["csa_64k"], "ds_fresh", (8191, 4095, 1023, 3), (1, 1, 1, 1), k=256),
    # FP8 indexer keys, MXFP4 pool
    "lp_fp8_keys": synth.shrink(S["lp_512k"], "ds_lp", (8191, 5002, 6003), (1, 1, 1), k=512),
    # indexers of 128 heads x 64 dims (one dimension per lane) and 32 x 256 (four)
    "idx128x64": synth.shrink(S["csa_64k"], "ds_i128", (4095, 3001, 2047), (1, 1, 1), k=256, HI=128, dI=64),
    "idx32x256": synth.shrink(S["csa_64k"], "ds_i32", (4095, 3001, 2047), (1, 1, 1), k=256, HI=32, dI=256),
    # rows over 32K entries: slices' top-k first, then the candidates beside compress_append
    "lp_two_launch": synth.shrink(S["lp_512k"], "ds_lp_long", (140003, 131071, 70000), (1, 1, 1), k=2048),
}


def _say(*a):
    print(*a, flush=True)


def _ld(c):
    return (c.max_entries + 3) // 4 * 4


def _separate(gs, ld):
    nr = len(gs.st.row_seq)
    gs.ld = ld
    gs.compress_append()
    lg = gs.index(logits=torch.zeros((nr, ld), dtype=torch.float32, device=DEV))
    return lg, gs.topk(lg)


def _fused(gs, ld):
    c = gs.cfg
    nr = len(gs.st.row_seq)
    lg = torch.zeros((nr, ld), dtype=torch.float32, device=DEV)
    idx = torch.empty((nr, c.k), dtype=torch.int32, device=DEV)
    ws = torch.zeros(lcca.decode_select_workspace_size(gs.rows, c.m, c.k), dtype=torch.uint8, device=DEV)
    for _ in range(2):
        # twice on the same workspace: the counts it holds must be back to
        # zero after each call (the step is idempotent at fixed positions)
        lcca.decode_select(gs.pages, gs.rows, gs.cu_new, gs.start_pos, int(gs.st.cu_new[-1]), gs.tok_ldt,
                           gs.new_kv, gs.new_kv_logit, gs.new_ik, gs.new_ik_logit, gs.kv, gs.ik, gs.win, gs.rem,
                           gs.q_dt, gs.q_idx, c.HI, gs.w_idx, 1.0, lg, ld, c.k, idx, ws)
        if c.max_entries <= 32768:
            torch.cuda.synchronize()
            assert not ws.any(), "leading-digit counts left in the workspace"
    return lg, idx


def _state_tensors(gs):
    out = {"kv": gs.kv.data, "ik": gs.ik.data, "win": gs.win.data, "rem_kv": gs.rem.kv, "rem_kv_logit": gs.rem.kv_logit,
           "rem_ik": gs.rem.ik, "rem_ik_logit": gs.rem.ik_logit}
    if gs.kv.scale is not None:
        out["kv_scale"] = gs.kv.scale
    if gs.win.scale is not None:
        out["win_scale"] = gs.win.scale
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_decode_select_equals_the_three_calls(name):
    cfg = CASES[name]
    _say("decode_select", name)
    st = State(cfg)
    ld = _ld(cfg)
    a, b = GpuState(st), GpuState(st)
    lg_a, idx_a = _separate(a, ld)
    lg_b, idx_b = _fused(b, ld)
    torch.cuda.synchronize()
    for key, ta in _state_tensors(a).items():
        tb = _state_tensors(b)[key]
        assert torch.equal(ta.view(torch.uint8), tb.view(torch.uint8)), key
    c = cfg
    m = c.m
    pos = st.row_pos.astype(np.int64)
    n_r = (pos + 1) // m
    fresh = (pos + 1) % m == 0
    assert fresh.any()
    la, lb = lg_a.cpu().numpy(), lg_b.cpu().numpy()
    q = O.bf16_decode(st.q_idx.reshape(len(pos), c.HI, c.dI)).astype(np.float64)
    ikh = a.ik.data.cpu().numpy()
    row_bytes = c.dI * (2 if c.ik_dtype == synth.BF16 else 1)
    for r in range(len(pos)):
        stop = n_r[r] - 1 if fresh[r] else n_r[r]
        assert np.array_equal(la[r, :stop].view(np.uint32), lb[r, :stop].view(np.uint32)), r
        assert not lb[r, n_r[r]:].any()
        if fresh[r]:
            g = n_r[r] - 1
            prow = int(pool_rows(st.bt, m, st.row_seq[r], [g])[0])
            raw = ikh[prow * row_bytes:(prow + 1) * row_bytes]
            k = (O.bf16_decode(raw.view(np.uint16)) if c.ik_dtype == synth.BF16 else O.fp8_decode(raw)).astype(np.float64)
            bound = float((st.w_idx[r].astype(np.float64) * (np.abs(q[r]) @ np.abs(k))).sum())
            exact = float((st.w_idx[r].astype(np.float64) * np.maximum(q[r] @ k, 0.0)).sum())
            assert abs(lb[r, g] - exact) <= 2e-5 * bound, (r, lb[r, g], exact, bound)
            assert abs(la[r, g] - lb[r, g]) <= 4e-5 * bound
    assert torch.equal(idx_a, idx_b)
    want = O.topk(st.row_pos, m, la.astype(np.float64), c.k)
    assert np.array_equal(idx_a.cpu().numpy(), want)


def test_rows_that_are_not_the_new_tokens_get_nan():
    """The device-side half of the contract: when a sequence does not append
    exactly one token at its row's position (here sequence 0 appends none and
    sequence 1 two, which the host cannot see), the entry a row's token
    would complete gets a NaN logit instead of a logit of stale pool bytes."""
    cfg = synth.shrink(S["csa_64k"], "ds_contract", (9999, 3003), (1, 1), k=256)
    _say("decode_select contract check")
    st = State(cfg)
    ld = _ld(cfg)
    gs = GpuState(st)
    gs.cu_new = torch.tensor([0, 0, 2], dtype=torch.int32, device=DEV)
    lg, _ = _fused(gs, ld)
    torch.cuda.synchronize()
    pos = st.row_pos.astype(np.int64)
    n_r = (pos + 1) // cfg.m
    assert ((pos + 1) % cfg.m == 0).all()
    lh = lg.cpu().numpy()
    for r in range(len(pos)):
        assert np.isnan(lh[r, n_r[r] - 1])
        assert np.isfinite(lh[r, : n_r[r] - 1]).all()
