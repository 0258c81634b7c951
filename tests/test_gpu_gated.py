"""lcca_compress_append_gated against the oracle's gated compress_append.

Every channel of every token has its own N(0,1) aggregation logit.  Pool
entries must be correct roundings of the oracle's fp64 aggregate within the
device's fp32 error bound eps = (m + 8) 2^-24 sum_i w_ic |x_ic| (per
channel, computed by the oracle on |x|), with at least 99.9% identical codes;
the window ring, the remainder ring's tokens and its per-channel logit rows
are bit-exact.  Cases: chunks starting inside a group (one whose first group
reads ring slots its tail rewrites), decode steps (one token per sequence),
MXFP4 / FP8 pools, fp32 tokens, and 128-token groups."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import compare as C
import oracle as O
from long_context_compressed_append_amd import lcca, synth
from state import State, pool_rows
from gpu_state import GpuState, dev_typed

pytestmark = pytest.mark.gpu

S = synth.CONFIGS
CASES = [
    synth.shrink(S["csa_64k"], "gated_csa", (3001, 1024, 502), (70, 90, 1), k=64),
    synth.shrink(S["csa_64k"], "gated_decode", (9999, 4101, 3003), (1, 1, 1), k=64),
    synth.shrink(S["lp_512k"], "gated_lp", (2047, 777), (100, 63), k=64),
    synth.shrink(S["tiny"], "gated_tiny", (0, 5), (100, 90), win_cap=2048),
    synth.shrink(S["hca_1m"], "gated_hca", (40959, 25600), (200, 130)),
    synth.shrink(S["hca_1m"], "gated_hca_decode", (40959, 25599, 777), (1, 1, 1)),
    # 16-token groups (the slice kernel) with a chunk whose first group reads
    # ring slots its tail rewrites
    synth.shrink(S["csa_64k"], "gated_m16", (3001, 1039), (70, 1), k=64, m=16),
]


def _gated(st: State):
    """The state's remainder-ring logits replaced by per-channel rows, and
    the new tokens' per-channel logits (kv [n][D], ik [n][dI] or None)."""
    c = st.cfg
    rk = np.zeros((c.batch * c.m, c.D), np.float32)
    ri = np.zeros((c.batch * c.m, max(c.dI, 1)), np.float32)
    nks, nis = [], []
    for b in range(c.batch):
        r_kv, r_ik, n_kv, n_ik = synth.gate_logits(c, b)
        t0 = (c.prior_len[b] // c.m) * c.m
        slots = b * c.m + (np.arange(t0, t0 + r_kv.shape[0]) % c.m)
        rk[slots] = r_kv
        nks.append(n_kv)
        if c.HI:
            ri[slots] = r_ik
            nis.append(n_ik)
    st.rem_kv_logit = rk.reshape(-1)
    st.rem_ik_logit = ri.reshape(-1)
    nk = np.concatenate(nks).astype(np.float32)
    ni = np.concatenate(nis).astype(np.float32) if c.HI else None
    return nk, ni


def _oracle(st, nk, ni):
    c = st.cfg
    O.compress_append(st.bt, st.cu_new, st.start_pos, st.tok_dt, st.new_kv, nk, st.new_ik if c.HI else None,
                      ni, c.m, c.D, c.dI, st.kv.as_dict(), st.ik.as_dict() if st.ik else None, st.win.as_dict(),
                      st.rem_dict(), gated=True)


def _abs_tokens(st):
    if st.cfg.tok_dtype == synth.F32:
        for a in (st.new_kv, st.new_ik, st.rem_kv.view(np.float32), st.rem_ik.view(np.float32)):
            if a is not None:
                np.abs(a, out=a)
    else:
        for a in (st.new_kv, st.new_ik, st.rem_kv.view(np.uint16), st.rem_ik.view(np.uint16)):
            if a is not None:
                a &= np.uint16(0x7FFF)


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_gated_compress_append_parity(cfg):
    print("gated compress_append", cfg.name, flush=True)
    st = State(cfg)
    nk, ni = _gated(st)
    g = GpuState(st)
    rem = lcca.Remainder(g.tok_ldt, g.rem.kv, dev_typed(st.rem_kv_logit), g.rem.ik if cfg.HI else None,
                         dev_typed(st.rem_ik_logit) if cfg.HI else None)
    lcca.compress_append_gated(g.pages, g.cu_new, g.start_pos, int(st.cu_new[-1]), g.tok_ldt, g.new_kv,
                               dev_typed(nk), g.new_ik, dev_typed(ni) if cfg.HI else None, g.kv, g.ik, g.win, rem)
    torch.cuda.synchronize()
    ora = st.copy_caches()
    _oracle(ora, nk, ni)
    f32cfg = replace(cfg, kv_dtype=synth.F32, ik_dtype=synth.F32)
    ex = State(f32cfg)
    ex_nk, ex_ni = _gated(ex)
    _oracle(ex, ex_nk, ex_ni)
    ab = State(f32cfg)
    ab_nk, ab_ni = _gated(ab)
    _abs_tokens(ab)
    _oracle(ab, ab_nk, ab_ni)
    rows = np.concatenate([pool_rows(st.bt, cfg.m, b, np.arange(cfg.prior_len[b] // cfg.m, cfg.total_len(b) // cfg.m))
                           for b in range(cfg.batch)])
    for what, gstore, ostore, dim in (("kv", g.kv, ora.kv, cfg.D), ("ik", g.ik, ora.ik, cfg.dI)):
        if gstore is None:
            continue
        gdata = gstore.data.cpu().numpy()
        gscale = gstore.scale.cpu().numpy() if gstore.scale is not None else None
        rb = O.row_bytes(ostore.dtype, dim)
        nrow = gdata.size // rb
        other = np.setdiff1d(np.arange(nrow), rows)
        assert np.array_equal(gdata.reshape(nrow, rb)[other], ostore.data.reshape(nrow, rb)[other]), what
        if len(rows) == 0:
            continue
        got = np.stack([O.load_rows(ostore.dtype, gdata, gscale, int(r), 1, dim)[0] for r in rows])
        exact = (ex.kv if what == "kv" else ex.ik).rows(rows)
        eps = (cfg.m + 8) * 2.0 ** -24 * (ab.kv if what == "kv" else ab.ik).rows(rows)
        gsc = gscale.reshape(nrow, -1)[rows] if gscale is not None and ostore.dtype == O.MXFP4 else None
        C.check_correct_rounding(ostore.dtype, got, exact, eps, gdata.reshape(nrow, rb)[rows],
                                 ostore.data.reshape(nrow, rb)[rows], dim, gsc)
    assert np.array_equal(g.win.data.cpu().numpy(), ora.win.data)
    if ora.win.scale is not None:
        assert np.array_equal(g.win.scale.cpu().numpy(), ora.win.scale)
    assert np.array_equal(g.rem.kv.cpu().numpy(), ora.rem_kv)
    assert np.array_equal(rem.kv_logit.cpu().numpy(), ora.rem_kv_logit)
    if cfg.HI:
        assert np.array_equal(g.rem.ik.cpu().numpy(), ora.rem_ik)
        assert np.array_equal(rem.ik_logit.cpu().numpy(), ora.rem_ik_logit)


def test_gated_with_uniform_logits_equals_the_per_token_call():
    """Channel-uniform logits: the gated kernel stores the per-token kernels'
    bytes up to the order of the sums (pools within one fp32 rounding step
    of each other's codes: compared through the oracle's bound above); the
    rings and window are identical."""
    cfg = CASES[0]
    st = State(cfg)
    g1 = GpuState(st.copy_caches())
    g1.compress_append()
    g2 = GpuState(st.copy_caches())
    c = cfg
    nk = np.repeat(st.new_kv_logit[:, None], c.D, 1).astype(np.float32)
    ni = np.repeat(st.new_ik_logit[:, None], c.dI, 1).astype(np.float32)
    rk = np.repeat(st.rem_kv_logit[:, None], c.D, 1).astype(np.float32)
    ri = np.repeat(st.rem_ik_logit[:, None], c.dI, 1).astype(np.float32)
    rem = lcca.Remainder(g2.tok_ldt, g2.rem.kv, dev_typed(rk.reshape(-1)), g2.rem.ik, dev_typed(ri.reshape(-1)))
    lcca.compress_append_gated(g2.pages, g2.cu_new, g2.start_pos, int(st.cu_new[-1]), g2.tok_ldt, g2.new_kv,
                               dev_typed(nk), g2.new_ik, dev_typed(ni), g2.kv, g2.ik, g2.win, rem)
    torch.cuda.synchronize()
    assert np.array_equal(g1.win.data.cpu().numpy(), g2.win.data.cpu().numpy())
    assert np.array_equal(g1.rem.kv.cpu().numpy(), g2.rem.kv.cpu().numpy())
    a = O.bf16_decode(g1.kv.data.cpu().numpy().view(np.uint16))
    b = O.bf16_decode(g2.kv.data.cpu().numpy().view(np.uint16))
    # bf16 codes of the same aggregate summed in another order: at most one
    # rounding step apart, and mostly identical
    assert np.all(np.abs(a - b) <= C.ulp_bf16(np.maximum(np.abs(a), np.abs(b))))
    assert (a != b).mean() < 0.01
