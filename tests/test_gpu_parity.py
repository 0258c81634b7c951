"""Parity of the device library with the oracle, stage by stage and end to
end, on reduced-size versions of every workload (several tiles, ragged
lengths, remainder rings in use) and on the full tiny workload.

Stage-isolated tests hand the device exactly the bytes the oracle stage
reads; end-to-end tests run both chains from the same initial state."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle as O
from long_context_compressed_append_amd import lcca, synth
from state import State, pool_rows
import compare as C

pytestmark = pytest.mark.gpu

S = synth.CONFIGS
SMALL = {
    "tiny": S["tiny"],
    "csa_small": synth.shrink(S["csa_64k"], "csa_small", (9999, 4101, 3003), (1, 1, 1), k=512),
    "hca_small": synth.shrink(S["hca_1m"], "hca_small", (40959, 25600), (1, 1)),
    "prefill_small": synth.shrink(S["prefill_8k"], "prefill_small", (3001,), (1000,), k=256, win_cap=2048),
    "lp_small": synth.shrink(S["lp_512k"], "lp_small", (8191, 5000), (1, 1), k=512),
    # other built shapes: 128 heads of dim 128 (two 64-head blocks) with a
    # 32 x 64 indexer; 128 x 64 and 32 x 256 indexers; an MXFP4 pool with a
    # bf16 window; many rows (no key splits) with 128 heads
    "h128_d128": synth.shrink(S["csa_64k"], "h128_d128", (5001, 2222), (1, 1), k=256, D=128, H=128, HI=32, dI=64),
    "idx128x64": synth.shrink(S["csa_64k"], "idx128x64", (4097, 3000), (1, 1), k=256, HI=128, dI=64),
    "idx32x256": synth.shrink(S["csa_64k"], "idx32x256", (4097, 3000), (1, 1), k=256, HI=32, dI=256),
    "lp_bf16win": synth.shrink(S["lp_512k"], "lp_bf16win", (6001, 3333), (1, 1), k=256, win_dtype=synth.BF16),
    "prefill_h128": synth.shrink(S["prefill_8k"], "prefill_h128", (2001,), (300,), k=128, win_cap=1024, H=128),
    # chunked prefill of three sequences (424 rows, not a multiple of 16):
    # indexer workgroups and waves hold rows of two sequences
    "prefill_multi": synth.shrink(S["prefill_8k"], "prefill_multi", (3001, 1500, 777), (203, 131, 90), k=256,
                                  win_cap=2048),
}


def _say(*a):
    print(*a, flush=True)


def _gpu(st):
    from gpu_state import GpuState
    return GpuState(st)


def _kind(cfg):
    if cfg.kv_dtype == synth.F32:
        return "f32"
    return "mxfp4" if cfg.kv_dtype == synth.MXFP4 else "bf16"


def _abs_tokens(st):
    """Replace every token value of a State by its absolute value."""
    if st.cfg.tok_dtype == synth.F32:
        for a in (st.new_kv, st.new_ik, st.rem_kv.view(np.float32), st.rem_ik.view(np.float32)):
            if a is not None:
                np.abs(a, out=a)
    else:
        for a in (st.new_kv, st.new_ik, st.rem_kv.view(np.uint16), st.rem_ik.view(np.uint16)):
            if a is not None:
                a &= np.uint16(0x7FFF)


def _written_rows(cfg, bt):
    rows = []
    for b in range(cfg.batch):
        s, e = cfg.prior_len[b], cfg.total_len(b)
        g = np.arange(s // cfg.m, e // cfg.m)
        rows.append(pool_rows(bt, cfg.m, b, g))
    return np.concatenate(rows) if rows else np.zeros(0, np.int64)


@pytest.mark.parametrize("name", list(SMALL))
def test_compress_append_parity(name):
    cfg = SMALL[name]
    _say("compress_append parity", name)
    st = State(cfg)
    gs = _gpu(st)
    gs.compress_append()
    torch.cuda.synchronize()
    ora = st.copy_caches()
    ora.oracle_compress_append()
    # fp32 values before encoding (oracle with f32 pools), and sum_i w_i |x_i|
    # (the same aggregation of the absolute token values) for the device's
    # fp32 error bound eps = (m + 8) * 2^-24 * sum_i w_i |x_i|
    f32cfg = replace(cfg, kv_dtype=synth.F32, ik_dtype=synth.F32)
    ex = State(f32cfg)
    ex.oracle_compress_append()
    ab = State(f32cfg)
    _abs_tokens(ab)
    ab.oracle_compress_append()
    rows = _written_rows(cfg, st.bt)
    for what, gstore, ostore, dim in (("kv", gs.kv, ora.kv, cfg.D), ("ik", gs.ik, ora.ik, cfg.dI)):
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
    # window ring and remainder ring: bit-exact
    assert np.array_equal(gs.win.data.cpu().numpy(), ora.win.data)
    if ora.win.scale is not None:
        assert np.array_equal(gs.win.scale.cpu().numpy(), ora.win.scale)
    assert np.array_equal(gs.rem.kv.cpu().numpy(), ora.rem_kv)
    assert np.array_equal(gs.rem.kv_logit.cpu().numpy(), ora.rem_kv_logit)
    if cfg.HI:
        assert np.array_equal(gs.rem.ik.cpu().numpy(), ora.rem_ik)
        assert np.array_equal(gs.rem.ik_logit.cpu().numpy(), ora.rem_ik_logit)


def _index_bound(st, rows):
    """sum_h w_h sum_d |q_hd k_d| for every visible entry of the given rows."""
    c = st.cfg
    out = np.zeros((len(rows), c.max_entries))
    q = st.q_idx.reshape(len(st.row_seq), c.HI, c.dI)
    qf = (O.bf16_decode(q) if c.q_dtype != synth.F32 else q.view(np.float32)).astype(np.float64)
    for i, r in enumerate(rows):
        b, n = st.row_seq[r], (st.row_pos[r] + 1) // c.m
        K = st.ik.rows(pool_rows(st.bt, c.m, b, np.arange(n)))
        out[i, :n] = (st.w_idx[r][:, None] * (np.abs(qf[r]) @ np.abs(K).T)).sum(0)
    return out


@pytest.mark.parametrize("name", [n for n in SMALL if SMALL[n].HI])
def test_index_topk_attention_stagewise(name):
    cfg = SMALL[name]
    _say("stagewise parity", name)
    st = State(cfg)
    st.oracle_compress_append()
    gs = _gpu(st)                                 # device gets the oracle's post-append caches
    nrows = len(st.row_seq)
    check = np.unique(np.r_[0:min(nrows, 24), max(0, nrows - 24):nrows])
    # indexer
    lg = gs.index()
    torch.cuda.synchronize()
    lg_h = lg.cpu().numpy()
    want = st.oracle_index(check)
    n_r = (st.row_pos[check] + 1) // cfg.m
    C.check_logits(lg_h[check], want, _index_bound(st, check), n_r)
    # top-k on identical logits: identical lists
    idx = gs.topk(lg)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    want_idx = O.topk(st.row_pos, cfg.m, lg_h.astype(np.float64), cfg.k)
    assert np.array_equal(idx_h, want_idx)
    # attention on identical indices
    out, lse = gs.attn(idx)
    torch.cuda.synchronize()
    o_want, l_want = st.oracle_attn(idx_h[check], check)
    C.check_attention(out.cpu().numpy()[check], o_want, _kind(cfg))
    assert np.abs(lse.cpu().numpy()[check] - l_want).max() <= (1e-5 if _kind(cfg) == "f32" else 1e-3)


@pytest.mark.parametrize("name", [n for n in SMALL if not SMALL[n].HI])
def test_dense_attention_stagewise(name):
    cfg = SMALL[name]
    _say("dense attention parity", name)
    st = State(cfg)
    st.oracle_compress_append()
    gs = _gpu(st)
    out, lse = gs.attn(None)
    torch.cuda.synchronize()
    o_want, l_want = st.oracle_attn(None)
    C.check_attention(out.cpu().numpy(), o_want, _kind(cfg))
    assert np.abs(lse.cpu().numpy() - l_want).max() <= 1e-3


@pytest.mark.parametrize("name", list(SMALL))
def test_end_to_end(name):
    cfg = SMALL[name]
    _say("end-to-end parity", name)
    st = State(cfg)
    gs = _gpu(st)
    gs.compress_append()
    if cfg.HI:
        lg = gs.index()
        idx = gs.topk(lg)
    else:
        idx = None
    out, lse = gs.attn(idx)
    torch.cuda.synchronize()
    st.oracle_compress_append()
    nrows = len(st.row_seq)
    check = np.unique(np.r_[0:min(nrows, 16), max(0, nrows - 16):nrows])
    if cfg.HI:
        ol = st.oracle_index(check)
        idx_h = idx.cpu().numpy()
        for i, r in enumerate(check):
            C.check_topk_band(idx_h[r], ol[i], (st.row_pos[r] + 1) // cfg.m, cfg.k)
        # attention given the device's selection, then against the oracle's own selection
        o_sel, _ = st.oracle_attn(idx_h[check], check)
        C.check_attention(out.cpu().numpy()[check], o_sel, _kind(cfg))
        o_ora, _ = st.oracle_attn(st.oracle_topk(ol, check), check)
        C.check_attention(out.cpu().numpy()[check], o_ora, _kind(cfg))
    else:
        o_ora, _ = st.oracle_attn(None, check)
        C.check_attention(out.cpu().numpy()[check], o_ora, _kind(cfg))


def test_bf16_output_and_value_dim_512():
    cfg = SMALL["csa_small"]
    _say("bf16 output / d_v=512")
    st = State(cfg)
    st.oracle_compress_append()
    gs = _gpu(st)
    idx = gs.topk(gs.index())
    out, _ = gs.attn(idx, out_dtype=lcca.BF16, d_v=512)
    torch.cuda.synchronize()
    o_want, _ = O.sparse_attn(st.row_seq, st.row_pos, cfg.m, st.bt, st.q_dt,
                              st.q.reshape(len(st.row_seq), cfg.H, cfg.D), cfg.H, cfg.D, 512, cfg.scale,
                              st.kv.as_dict(), idx.cpu().numpy(), cfg.k, st.win.as_dict(), cfg.window)
    C.check_attention(out.float().cpu().numpy(), o_want, "bf16", out_bf16=True)


def test_bf16_output_split_partials_keep_their_range():
    """Key splits with bf16 outputs keep their partial states as fp16 with a
    power-of-two range scale.  Scaling the cache by 2^12 while dividing
    sm_scale by 2^12 leaves every score unchanged, so the outputs must scale
    by exactly 2^12 (bit for bit) and the lse stay the same; the scaled
    values (up to ~1e5) are beyond fp16's range without the scale."""
    cfg = SMALL["csa_small"]
    _say("split partial range (bf16 output)")
    st = State(cfg)
    st.oracle_compress_append()
    gs = _gpu(st)
    idx = gs.topk(gs.index())
    out1, lse1 = gs.attn(idx, out_dtype=lcca.BF16)
    big = st.copy_caches()
    big.kv.data[:] = O.bf16_encode(O.bf16_decode(big.kv.data.view(np.uint16)).astype(np.float32) * 4096.0).view(np.uint8)
    big.win.scale[:] = big.win.scale * np.float32(4096.0)
    gb = _gpu(big)
    nr = len(st.row_seq)
    out2 = torch.empty((nr, cfg.H, cfg.dv), dtype=torch.bfloat16, device="cuda")
    lse2 = torch.empty((nr, cfg.H), dtype=torch.float32, device="cuda")
    ws = gb.attn_workspace(idx) if hasattr(gb, "attn_workspace") else None
    if ws is None:
        wsb = lcca.sparse_attn_workspace_size(gb.rows, cfg.m, cfg.H, cfg.D, cfg.dv, cfg.k, True, cfg.window)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    lcca.sparse_attn_fwd(gb.pages, gb.rows, gb.q_dt, gb.q, cfg.H, cfg.dv, cfg.scale / 4096.0, gb.kv, idx, cfg.k, gb.win,
                         lcca.BF16, out2, lse2, ws)
    torch.cuda.synchronize()
    a = out1.float().cpu().numpy() * 4096.0
    b = out2.float().cpu().numpy()
    assert np.isfinite(b).all()
    assert np.array_equal(a, b)
    assert np.array_equal(lse1.cpu().numpy(), lse2.cpu().numpy())
