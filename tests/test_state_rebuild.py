"""Single-layer state rebuild on the oracle (see tests/rebuild.py): rings
overwritten with junk and rebuilt by replaying from a group boundary give
the same entries, ring contents and decode outputs as the uninterrupted
history, bit for bit; a replay that starts inside a group does not (its
first group would be formed from the junk remainder ring)."""
import numpy as np
import pytest

import oracle as O
from rebuild import JUNK, STEPS, Scenario


def _run(sc, replay):
    """Oracle history, optional junk + replay of `replay` ranges, two decode steps."""
    c = sc.cfg
    st = sc.st.copy_caches()
    st.oracle_compress_append(*sc.tokens(sc.history()))
    if replay is not None:
        st.win.data[:] = JUNK
        if st.win.scale is not None:
            st.win.scale[:] = 3.0
        st.rem_kv[:] = JUNK
        st.rem_ik[:] = JUNK
        st.rem_kv_logit[:] = 5.0
        st.rem_ik_logit[:] = 5.0
        st.oracle_compress_append(*sc.tokens(replay))
    outs = []
    for s in range(STEPS):
        st.oracle_compress_append(*sc.tokens(sc.step_tokens(s)))
        rs, rp = sc.rows(s)
        lg = idx = None
        if c.HI:
            lg = O.index_logits(rs, rp, c.m, st.bt, st.q_dt, sc.q_idx[s], c.HI, c.dI, sc.w_idx[s], 1.0,
                                st.ik.as_dict(), sc.ld)
            idx = O.topk(rp, c.m, lg, c.k)
        o, l = O.sparse_attn(rs, rp, c.m, st.bt, st.q_dt, sc.q[s], c.H, c.D, c.dv, c.scale, st.kv.as_dict(), idx,
                             c.k if idx is not None else 0, st.win.as_dict(), c.window)
        outs.append((lg, idx, o, l))
    return st, outs


def _same_state(a, b, sc):
    c = sc.cfg
    assert np.array_equal(a.kv.data, b.kv.data)
    if a.kv.scale is not None:
        assert np.array_equal(a.kv.scale, b.kv.scale)
    if c.HI:
        assert np.array_equal(a.ik.data, b.ik.data)
    ws = sc.live_window_slots()
    rb = O.row_bytes(a.win.dtype, c.D)
    assert np.array_equal(a.win.data.reshape(-1, rb)[ws], b.win.data.reshape(-1, rb)[ws])
    if a.win.scale is not None:
        assert np.array_equal(a.win.scale[ws], b.win.scale[ws])
    rs = sc.live_remainder_slots()
    tb = sc.tb
    assert np.array_equal(a.rem_kv.reshape(c.batch * c.m, -1)[rs], b.rem_kv.reshape(c.batch * c.m, -1)[rs])
    assert np.array_equal(a.rem_kv_logit[rs], b.rem_kv_logit[rs])
    if c.HI:
        assert np.array_equal(a.rem_ik.reshape(c.batch * c.m, -1)[rs], b.rem_ik.reshape(c.batch * c.m, -1)[rs])
        assert np.array_equal(a.rem_ik_logit[rs], b.rem_ik_logit[rs])


@pytest.mark.parametrize("name", ["csa", "hca"])
def test_rebuild_equals_uninterrupted(name):
    sc = Scenario(name)
    a, out_a = _run(sc, None)
    b, out_b = _run(sc, sc.replay())
    _same_state(a, b, sc)
    for (la, ia, oa, sa), (lb, ib, ob, sb) in zip(out_a, out_b):
        if la is not None:
            assert np.array_equal(la, lb) and np.array_equal(ia, ib)
        assert np.array_equal(oa, ob) and np.array_equal(sa, sb)


def test_replay_inside_a_group_differs():
    sc = Scenario("csa")
    a, _ = _run(sc, None)
    ranges = [(s + 1, e) for s, e in sc.replay()]          # one past the boundary: inside a group
    b, _ = _run(sc, ranges)
    assert not np.array_equal(a.kv.data, b.kv.data)
