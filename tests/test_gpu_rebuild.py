"""Single-layer state rebuild on the device (see tests/rebuild.py): with the
rings overwritten with junk and rebuilt by replaying from a group boundary,
the device's entries, live ring slots and decode outputs equal those of the
uninterrupted device history bit for bit, and the decode outputs match the
oracle's uninterrupted history."""
import numpy as np
import pytest
import torch

import oracle as O
import compare as C
from long_context_compressed_append_amd import lcca
from rebuild import JUNK, STEPS, Scenario
from gpu_state import GpuState, dev_bytes, dev_typed

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _compress(gs, sc, ranges):
    c = sc.cfg
    cu, sp, kv, ka, ik, ia = sc.tokens(ranges)
    lcca.compress_append(gs.pages, dev_typed(cu), dev_typed(sp), int(cu[-1]), gs.tok_ldt, dev_bytes(kv),
                         dev_typed(ka), dev_bytes(ik) if c.HI else None, dev_typed(ia) if c.HI else None,
                         gs.kv, gs.ik, gs.win, gs.rem)


def _run(sc, rebuild):
    c = sc.cfg
    gs = GpuState(sc.st.copy_caches())
    _compress(gs, sc, sc.history())
    if rebuild:
        gs.win.data.fill_(JUNK)
        if gs.win.scale is not None:
            gs.win.scale.fill_(3.0)
        for t in (gs.rem.kv, gs.rem.ik):
            if t is not None:
                t.fill_(JUNK)
        for t in (gs.rem.kv_logit, gs.rem.ik_logit):
            if t is not None:
                t.fill_(5.0)
        _compress(gs, sc, sc.replay())
    outs = []
    for s in range(STEPS):
        _compress(gs, sc, sc.step_tokens(s))
        rs, rp = sc.rows(s)
        rows = lcca.Rows(dev_typed(rs), dev_typed(rp), int(rp.max()))
        idx = None
        lg = None
        if c.HI:
            lg = torch.zeros((c.batch, sc.ld), dtype=torch.float32, device="cuda")
            lcca.index_logits(gs.pages, rows, gs.q_dt, dev_bytes(sc.q_idx[s]), c.HI, dev_typed(sc.w_idx[s]), 1.0,
                              gs.ik, lg, sc.ld)
            idx = torch.empty((c.batch, c.k), dtype=torch.int32, device="cuda")
            wsb = lcca.topk_workspace_size(rows, c.m, c.k)
            tws = torch.empty(wsb, dtype=torch.uint8, device="cuda") if wsb else None
            lcca.topk_select(rows, c.m, lg, sc.ld, c.k, idx, tws)
        out = torch.empty((c.batch, c.H, c.dv), dtype=torch.float32, device="cuda")
        lse = torch.empty((c.batch, c.H), dtype=torch.float32, device="cuda")
        wsb = lcca.sparse_attn_workspace_size(rows, c.m, c.H, c.D, c.dv, c.k, idx is not None, c.window)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        lcca.sparse_attn_fwd(gs.pages, rows, gs.q_dt, dev_bytes(sc.q[s]), c.H, c.dv, c.scale, gs.kv, idx,
                             c.k if idx is not None else 0, gs.win, lcca.F32, out, lse, ws)
        torch.cuda.synchronize()
        outs.append(tuple(None if t is None else t.cpu().numpy() for t in (lg, idx, out, lse)))
    return gs, outs


@pytest.mark.parametrize("name", ["csa", "hca"])
def test_device_rebuild_equals_uninterrupted(name):
    _say("state rebuild", name)
    sc = Scenario(name)
    c = sc.cfg
    a, out_a = _run(sc, False)
    b, out_b = _run(sc, True)
    assert torch.equal(a.kv.data, b.kv.data)
    if a.kv.scale is not None:
        assert torch.equal(a.kv.scale, b.kv.scale)
    if c.HI:
        assert torch.equal(a.ik.data, b.ik.data)
    ws = torch.from_numpy(sc.live_window_slots()).cuda()
    wa, wb = a.win.data.view(c.batch * c.win_cap, -1), b.win.data.view(c.batch * c.win_cap, -1)
    assert torch.equal(wa[ws], wb[ws])
    if a.win.scale is not None:
        assert torch.equal(a.win.scale[ws], b.win.scale[ws])
    rs = torch.from_numpy(sc.live_remainder_slots()).cuda()
    assert torch.equal(a.rem.kv.view(c.batch * c.m, -1)[rs], b.rem.kv.view(c.batch * c.m, -1)[rs])
    assert torch.equal(a.rem.kv_logit[rs], b.rem.kv_logit[rs])
    for xa, xb in zip(out_a, out_b):
        for u, v in zip(xa, xb):
            if u is not None:
                assert np.array_equal(u, v)
    # the uninterrupted device history against the oracle's
    st = sc.st.copy_caches()
    st.oracle_compress_append(*sc.tokens(sc.history()))
    for s in range(STEPS):
        st.oracle_compress_append(*sc.tokens(sc.step_tokens(s)))
        rs_, rp = sc.rows(s)
        lg, idx, out, _ = out_a[s]
        if c.HI:
            ol = O.index_logits(rs_, rp, c.m, st.bt, st.q_dt, sc.q_idx[s], c.HI, c.dI, sc.w_idx[s], 1.0,
                                st.ik.as_dict(), sc.ld)
            for i in range(c.batch):
                C.check_topk_band(idx[i], ol[i], (int(rp[i]) + 1) // c.m, c.k)
        want, _ = O.sparse_attn(rs_, rp, c.m, st.bt, st.q_dt, sc.q[s], c.H, c.D, c.dv, c.scale, st.kv.as_dict(),
                                idx, c.k if idx is not None else 0, st.win.as_dict(), c.window)
        C.check_attention(out, want, "bf16")
