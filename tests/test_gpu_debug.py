"""The debug library (liblcca_debug.so, every kernel built with LCCA_DEBUG).

On valid inputs its calls store exactly the release library's bytes and
lcca_debug_check reports nothing.  Device-side indices outside their
contract -- a block-table entry outside the pool, a row's sequence outside
the batch or its position beyond max_pos, a compress_append chunk whose
cu_new / start_pos break the contract -- are each reported with their own
bit, and the word is clear again after the check.  The bad values are
written into the caller's own device arrays; the debug kernels replace
them by in-range values before any address is formed, so every access stays
inside the buffers and every kernel finishes."""
import numpy as np
import pytest
import torch

from long_context_compressed_append_amd import lcca, synth
from state import State
from gpu_state import GpuState, dev_typed

pytestmark = pytest.mark.gpu

S = synth.CONFIGS
# decode rows (one per sequence) over chunks that take the chunk kernel
DECODE = synth.shrink(S["csa_64k"], "dbg_decode", (3001, 1024), (70, 90), k=64)
# prefill rows (every new position) of a small chunk, so the slice kernel
# and the prefill indexer run
PREFILL = synth.shrink(S["prefill_8k"], "dbg_prefill", (1500,), (40,), k=64, win_cap=2048)


@pytest.fixture
def debug_lib():
    lcca.use_debug_library(True)
    assert "LCCA_DEBUG" in lcca.version()
    lcca.debug_check()                       # start from a clear word
    yield
    lcca.use_debug_library(False)


def _step(g: GpuState, out_dtype):
    g.compress_append()
    logits = g.index()
    idx = g.topk(logits)
    out, lse = g.attn(idx, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return [g.kv.data, g.win.data, g.rem.kv, g.rem.kv_logit] + ([g.ik.data] if g.ik is not None else []) + \
        ([g.kv.scale] if g.kv.scale is not None else []) + [logits, idx, out, lse]


@pytest.mark.parametrize("cfg,out_dtype", [(DECODE, lcca.BF16), (PREFILL, lcca.F32)], ids=["decode", "prefill"])
def test_debug_library_matches_release_on_valid_inputs(cfg, out_dtype):
    print("debug library vs release", cfg.name, flush=True)
    st = State(cfg)
    rel = _step(GpuState(st.copy_caches()), out_dtype)
    lcca.use_debug_library(True)
    try:
        lcca.debug_check()                   # start from a clear word
        dbg = _step(GpuState(st.copy_caches()), out_dtype)
        assert lcca.debug_check() == 0
    finally:
        lcca.use_debug_library(False)
    for i, (a, b) in enumerate(zip(rel, dbg)):
        a = a.cpu().contiguous().view(torch.uint8).numpy()
        b = b.cpu().contiguous().view(torch.uint8).numpy()
        assert np.array_equal(a, b), "output %d differs in %d bytes" % (i, int((a != b).sum()))


def _expect(bits):
    torch.cuda.synchronize()
    got = lcca.debug_check()
    assert got == bits, "error word %#x, expected %#x" % (got, bits)
    assert lcca.debug_check() == 0          # cleared by the check


def test_block_table_entry_outside_the_pool(debug_lib):
    print("debug: block-table entries", flush=True)
    st = State(DECODE)
    g = GpuState(st)
    c = DECODE
    good = g.pages.block_table.clone()
    # entry 0 of sequence 0 (visible to its row) lives in block 0
    g.pages.block_table[0, 0] = c.num_blocks + 5
    logits = g.index()
    _expect(lcca.DBG_BLOCK)
    idx = g.topk(logits)
    _expect(0)                               # the selection reads no block table
    idx[0, 0] = 0                            # make the row attend entry 0
    g.attn(idx)
    _expect(lcca.DBG_BLOCK)
    g.pages.block_table.copy_(good)
    # the block sequence 0's chunk completes its groups in
    blk = (c.prior_len[0] // c.m) // c.E
    g.pages.block_table[0, blk] = -3
    g.compress_append()
    _expect(lcca.DBG_BLOCK)
    g.pages.block_table.copy_(good)
    g.index()
    _expect(0)


def test_rows_outside_batch_or_max_pos(debug_lib):
    print("debug: rows", flush=True)
    st = State(DECODE)
    g = GpuState(st)
    logits = g.index()
    idx = g.topk(logits)
    _expect(0)
    pos = g.rows.row_pos.clone()
    g.rows.row_pos[1] = g.rows.max_pos + 100
    g.index(logits=logits)
    _expect(lcca.DBG_ROW)
    g.topk(logits, idx)
    _expect(lcca.DBG_ROW)
    g.attn(idx)
    _expect(lcca.DBG_ROW)
    g.rows.row_pos.copy_(pos)
    g.rows.row_pos[0] = -1
    g.attn(idx)
    _expect(lcca.DBG_ROW)
    g.rows.row_pos.copy_(pos)
    g.rows.row_seq[0] = DECODE.batch        # one past the last sequence
    g.index(logits=logits)
    _expect(lcca.DBG_ROW)
    g.attn(idx)
    _expect(lcca.DBG_ROW)


@pytest.mark.parametrize("cfg", [DECODE, PREFILL], ids=["chunk_kernel", "slice_kernel"])
def test_chunks_outside_their_contract(debug_lib, cfg):
    print("debug: chunks", cfg.name, flush=True)
    st = State(cfg)
    cu, sp = st.cu_new.copy(), st.start_pos.copy()
    cases = []
    bad = cu.copy(); bad[0] = 3                                    # cu_new[0] != 0
    cases.append((bad, sp))
    bad = sp.copy(); bad[-1] = -7                                  # negative start
    cases.append((cu, bad))
    bad = sp.copy(); bad[0] = cfg.max_blocks * 256 - 5             # chunk ends beyond the block table
    cases.append((cu, bad))
    if cfg.batch > 1:
        bad = cu.copy(); bad[1] = cu[2] + 3                        # decreasing, and beyond total_new
        cases.append((bad, sp))
    for bcu, bsp in cases:
        g = GpuState(st.copy_caches())
        g.cu_new = dev_typed(bcu.astype(np.int32))
        g.start_pos = dev_typed(bsp.astype(np.int32))
        g.compress_append()
        _expect(lcca.DBG_CHUNK)
    g = GpuState(st.copy_caches())
    g.compress_append()
    _expect(0)
