"""Attention with the softmax weights carried as bf16 alone
(q_dtype | LCCA_P_BF16) against the default hi + lo pair.

Each weight then differs from the pair's by at most 2^-9 of itself, so every
output element moves by at most 2^-9 max_j |v_j| (the largest value
component among the keys; bounded here by the pool's and window's largest)
plus fp32 rounding; lse is formed from the unrounded weights and stays bit
for bit.  Shapes: csa_64k with its outlier channels (the case the pair is
kept for), chunked prefill, an MXFP4 pool with an FP8 window; for the
prefill shape (N(0,1) values) also the oracle's bf16-path bounds."""
import numpy as np
import pytest
import torch

import compare as C
import oracle as O
from long_context_compressed_append_amd import lcca, synth
from state import State
from gpu_state import GpuState

pytestmark = pytest.mark.gpu

S = synth.CONFIGS
CASES = [
    synth.shrink(S["csa_64k"], "p16_csa", (9999, 4101, 3003), (1, 1, 1), k=512),
    synth.shrink(S["prefill_8k"], "p16_prefill", (3001,), (700,), k=256, win_cap=1024),
    synth.shrink(S["lp_512k"], "p16_lp", (8191, 5000), (1, 1), k=512),
]


def _max_value(st):
    c = st.cfg
    pool = np.abs(st.kv.rows(np.arange(c.num_blocks * c.E))[:, :c.dv]).max()
    win = np.abs(st.win.rows(np.arange(c.batch * c.win_cap))[:, :c.dv]).max()
    return max(pool, win)


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_bf16_weights_within_their_bound(cfg):
    print("bf16-only P", cfg.name, flush=True)
    st = State(cfg)
    st.oracle_compress_append()
    rows = np.arange(len(st.row_seq))
    idx = O.topk(st.row_pos, cfg.m, st.oracle_index(rows), cfg.k)
    gs = GpuState(st)
    idx_d = torch.from_numpy(idx).to("cuda")
    out_full, lse_full = gs.attn(idx_d)
    gs.q_dt = lcca.BF16 | lcca.P_BF16
    out_p16, lse_p16 = gs.attn(idx_d)
    torch.cuda.synchronize()
    assert torch.equal(lse_p16, lse_full)
    vmax = _max_value(st)
    d = np.abs(out_p16.cpu().numpy().astype(np.float64) - out_full.cpu().numpy())
    print("max |v| %.3g, max change %.3g (bound %.3g)" % (vmax, d.max(), 2.0 ** -9 * vmax), flush=True)
    assert np.all(d <= 2.0 ** -9 * vmax + 1e-6)
    if cfg.outlier_frac == 0.0:
        o_want, _ = st.oracle_attn(idx)
        C.check_attention(out_p16.cpu().numpy(), o_want, "mxfp4" if cfg.kv_dtype == synth.MXFP4 else "bf16")


def test_bf16_weights_with_bf16_outputs_and_noalloc():
    """The flag with bf16 outputs (fp16 split partials) within the same bound
    plus the bf16 output rounding of the default's result, and the
    allocation-free entry point with the flag equal to the workspace call bit
    for bit."""
    cfg = CASES[0]
    st = State(cfg)
    st.oracle_compress_append()
    rows = np.arange(len(st.row_seq))
    idx = O.topk(st.row_pos, cfg.m, st.oracle_index(rows), cfg.k)
    gs = GpuState(st)
    idx_d = torch.from_numpy(idx).to("cuda")
    out_full, _ = gs.attn(idx_d)
    qdt = lcca.BF16 | lcca.P_BF16
    gs.q_dt = qdt
    out_b, _ = gs.attn(idx_d, out_dtype=lcca.BF16)
    out_f, lse_f = gs.attn(idx_d)
    out_n = torch.empty_like(out_f)
    lse_n = torch.empty_like(lse_f)
    lcca.sparse_attn_fwd_noalloc(gs.pages, gs.rows, qdt, gs.q, cfg.H, cfg.dv, cfg.scale, gs.kv, idx_d, cfg.k, gs.win,
                                 lcca.F32, out_n, lse_n)
    torch.cuda.synchronize()
    assert torch.equal(out_n, out_f) and torch.equal(lse_n, lse_f)
    full = out_full.cpu().numpy().astype(np.float64)
    got = out_b.float().cpu().numpy().astype(np.float64)
    # bf16 output: half an ulp of the value (2^-9 relative) on top of the
    # weights' bound and the fp16 partials' 2^-12 of each 16-dim tile's range
    vmax = _max_value(st)
    bound = 2.0 ** -9 * vmax + 2.0 ** -9 * np.abs(full) + 2.0 ** -11 * vmax + 1e-6
    d = np.abs(got - full)
    print("bf16 outputs: max change %.3g (max |v| %.3g)" % (d.max(), vmax), flush=True)
    assert np.all(d <= bound)
