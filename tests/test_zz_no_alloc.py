"""lcca_sparse_attn_fwd_noalloc (the allocation-free entry point) against
lcca_sparse_attn_fwd on the same inputs, through the C ABI: two calls in a row,
the second with fewer rows, each output, lse and the oracle's bound checked.
The two entry points run the same kernels with the same split plan, so their
outputs must agree bit for bit; the first call's partial states are still in
the scratch array when the second runs."""
import numpy as np
import pytest
import torch

import compare as C
from long_context_compressed_append_amd import lcca, synth
from state import State
from gpu_state import GpuState, dev_typed

pytestmark = pytest.mark.gpu

S = synth.CONFIGS
CASES = [
    # rows of 10K and 4K positions with top-k 512: key splits, bf16 and fp32 outputs
    synth.shrink(S["csa_64k"], "noalloc_csa", (9999, 4101, 3003, 7777), (1, 1, 1, 1), k=512),
    # dense HCA rows (many tiles per row): more splits
    synth.shrink(S["hca_1m"], "noalloc_hca", (40959, 25600, 11111), (1, 1, 1)),
]


def _attn_pair(gs, cfg, idx, rows, out_dtype):
    """(out, lse) of both entry points for the first `rows` rows."""
    nr = rows
    sub = lcca.Rows(gs.rows.row_seq[:nr].contiguous(), gs.rows.row_pos[:nr].contiguous(),
                    int(gs.st.row_pos[:nr].max()))
    tdt = torch.float32 if out_dtype == lcca.F32 else torch.bfloat16
    res = []
    for noalloc in (False, True):
        out = torch.full((nr, cfg.H, cfg.dv), 7.0, dtype=tdt, device="cuda")
        lse = torch.full((nr, cfg.H), 7.0, dtype=torch.float32, device="cuda")
        sel = idx[:nr].contiguous() if idx is not None else None
        k = cfg.k if idx is not None else 0
        if noalloc:
            lcca.sparse_attn_fwd_noalloc(gs.pages, sub, gs.q_dt, gs.q, cfg.H, cfg.dv, cfg.scale, gs.kv, sel, k,
                                         gs.win, out_dtype, out, lse)
        else:
            wsb = lcca.sparse_attn_workspace_size(sub, cfg.m, cfg.H, cfg.D, cfg.dv, cfg.k, idx is not None,
                                                  cfg.window)
            assert wsb > 0, "the case must use key splits"
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            lcca.sparse_attn_fwd(gs.pages, sub, gs.q_dt, gs.q, cfg.H, cfg.dv, cfg.scale, gs.kv, sel, k, gs.win,
                                 out_dtype, out, lse, ws)
        res.append((out, lse))
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
@pytest.mark.parametrize("out_dtype", [lcca.F32, lcca.BF16], ids=["f32", "bf16"])
def test_noalloc_matches_workspace_entry(cfg, out_dtype):
    print("noalloc", cfg.name, out_dtype, flush=True)
    st = State(cfg)
    st.oracle_compress_append()
    gs = GpuState(st)
    idx = None
    if cfg.HI:
        idx = gs.topk(gs.index())
    nrows = len(st.row_seq)
    for rows in (nrows, nrows - 1):                 # two calls, the second smaller
        (o1, l1), (o2, l2) = _attn_pair(gs, cfg, idx, rows, out_dtype)
        a = o1.float().cpu().numpy()
        b = o2.float().cpu().numpy()
        assert np.array_equal(a, b), "outputs differ (max %.3g)" % np.abs(a - b).max()
        assert np.array_equal(l1.cpu().numpy(), l2.cpu().numpy())
        want, _ = st.oracle_attn(idx.cpu().numpy()[:rows] if idx is not None else None, np.arange(rows))
        C.check_attention(b, want, "bf16", out_bf16=out_dtype == lcca.BF16)
