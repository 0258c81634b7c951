"""Attention with FP8 queries on an MXFP4 pool (q_dtype | LCCA_Q_FP8).

Each (row, head) query is quantised to E4M3 with one power-of-two scale
(the rule of orc_quantize_fp8_rows); pool tiles are scored by the scaled
FP4 x FP8 MFMA on the pool's own codes and scales, window tiles by bf16
MFMAs on the dequantised query, so every key sees the same query q~.

* Parity: the device output equals the oracle's attention with q~
  (dequantised exactly, passed as fp32) within max-abs 1e-4 and mean-abs
  1e-5: the weights travel as a bf16 hi + lo pair (16 significant bits),
  so an output moves by at most about 2^-16 max|v| (6e-5 for |v| <= 4)
  plus fp32 rounding; lse within 1e-5 (measured about 2e-6).
* Against the unquantised query (the oracle with the bf16 q), the FP8
  variant's own tolerance: max-abs 5e-2 and mean-abs 5e-3.  A query element
  moves by up to 2^-4 of its value (RMS about 2.8 % for N(0,1) entries), so a
  score s = q.k / sqrt(D) moves by about 0.028 (RMS); the output, a softmax
  average over ~2K keys with sqrt(sum p^2) about 0.035, moves by about 1e-3
  (RMS).  Relative L2 is not asked: the outputs are themselves averages of
  magnitude ~|v| sqrt(sum p^2), so 1e-3 is a few percent of their norm.
Shapes: the lp_512k attention (64 heads x 576, FP8 window) over several
splits per row, d_v = 512, a bf16 window, and D = 128; one head of one row
is all zeros (X = -127), one row has fewer visible entries than k (masked
slots in its pool tiles)."""
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
    synth.shrink(S["lp_512k"], "q8a_lp", (8191, 5002, 6003, 100), (1, 1, 1, 1), k=512),
    synth.shrink(S["lp_512k"], "q8a_dv512", (4095, 3001), (1, 1), k=256, d_v=512),
    synth.shrink(S["lp_512k"], "q8a_bf16win", (4095, 3001, 2047), (1, 1, 1), k=256, win_dtype=synth.BF16),
    synth.shrink(S["lp_512k"], "q8a_d128", (4095, 3001), (1, 1), k=256, D=128),
]
Q8 = lcca.BF16 | lcca.Q_FP8


def _state(cfg):
    st = State(cfg)
    q = st.q.reshape(len(st.row_seq), cfg.H, cfg.D)
    q[0, 3, :] = 0                                    # a zero head
    st.oracle_compress_append()
    return st


def _quantised(st):
    c = st.cfg
    nr = len(st.row_seq)
    qf = O.bf16_decode(st.q).astype(np.float32).reshape(nr * c.H, c.D)
    codes, X = O.quantize_fp8_rows(qf)
    qd = (O.fp8_decode(codes) * 2.0 ** X[:, None].astype(np.float64)).astype(np.float32)
    return qd.reshape(nr, c.H, c.D), X.reshape(nr, c.H)


def _oracle_attn(st, idx, q_dtype, q):
    c = st.cfg
    return O.sparse_attn(st.row_seq, st.row_pos, c.m, st.bt, q_dtype, q, c.H, c.D, c.dv, c.scale, st.kv.as_dict(),
                         idx, c.k, st.win.as_dict(), c.window)


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_fp8_query_attention_parity(cfg):
    print("fp8-query attention", cfg.name, flush=True)
    st = _state(cfg)
    rows = np.arange(len(st.row_seq))
    lg = st.oracle_index(rows)
    idx = O.topk(st.row_pos, cfg.m, lg, cfg.k)
    gs = GpuState(st)
    gs.q_dt = Q8
    out, lse = gs.attn(torch.from_numpy(idx).to("cuda"))
    torch.cuda.synchronize()
    got, got_lse = out.cpu().numpy(), lse.cpu().numpy()
    qd, X = _quantised(st)
    assert X[0, 3] == -127
    o_q8, l_q8 = _oracle_attn(st, idx, O.F32, qd)
    d = np.abs(got.astype(np.float64) - o_q8)
    print("device vs oracle(q~): max %.3g mean %.3g, lse max %.3g"
          % (d.max(), d.mean(), np.abs(got_lse - l_q8).max()), flush=True)
    assert d.max() <= 1e-4 and d.mean() <= 1e-5
    assert np.abs(got_lse - l_q8).max() <= 1e-5
    # against the unquantised query
    o_bf, l_bf = _oracle_attn(st, idx, O.BF16, st.q.reshape(len(rows), cfg.H, cfg.D))
    qe = np.abs(o_q8 - o_bf)
    rel = np.linalg.norm(o_q8 - o_bf) / np.linalg.norm(o_bf)
    print("quantisation effect on the outputs: max %.3g mean %.3g rel-L2 %.3g, lse max %.3g"
          % (qe.max(), qe.mean(), rel, np.abs(l_q8 - l_bf).max()), flush=True)
    e = np.abs(got.astype(np.float64) - o_bf)
    assert e.max() <= 5e-2 and e.mean() <= 5e-3, (e.max(), e.mean())


def test_fp8_query_attention_rejected_without_mxfp4_pool():
    cfg = synth.shrink(S["csa_64k"], "q8a_bf16pool", (4095,), (1,), k=256)
    st = State(cfg)
    gs = GpuState(st)
    gs.q_dt = Q8
    with pytest.raises(lcca.LccaError) as e:
        gs.attn(None)
    assert e.value.status == lcca.ERR_UNSUPPORTED


def test_fp8_query_attention_bf16_outputs_and_noalloc():
    """The same FP8-query attention with bf16 outputs (fp16 split partials)
    against the oracle with q~ at the bf16-output bound, and the allocation-
    free entry point with fp32 outputs equal to the workspace call bit for
    bit."""
    cfg = CASES[0]
    st = _state(cfg)
    rows = np.arange(len(st.row_seq))
    idx = O.topk(st.row_pos, cfg.m, st.oracle_index(rows), cfg.k)
    gs = GpuState(st)
    gs.q_dt = Q8
    idx_d = torch.from_numpy(idx).to("cuda")
    qd, _ = _quantised(st)
    o_q8, _ = _oracle_attn(st, idx, O.F32, qd)
    out_b, _ = gs.attn(idx_d, out_dtype=lcca.BF16)
    out_f, lse_f = gs.attn(idx_d)
    out_n = torch.empty_like(out_f)
    lse_n = torch.empty_like(lse_f)
    lcca.sparse_attn_fwd_noalloc(gs.pages, gs.rows, Q8, gs.q, cfg.H, cfg.dv, cfg.scale, gs.kv, idx_d, cfg.k, gs.win,
                                 lcca.F32, out_n, lse_n)
    torch.cuda.synchronize()
    C.check_attention(out_b.float().cpu().numpy(), o_q8, "mxfp4", out_bf16=True)
    assert torch.equal(out_n, out_f) and torch.equal(lse_n, lse_f)
