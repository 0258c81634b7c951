"""compress_append's two launch shapes store the same bytes: one call
appending chunks of several sequences (the chunk kernel: 16 new tokens per
workgroup) against the same tokens appended sequence by sequence in halves of
fewer than 64 tokens (the slice kernel).  Pools, window ring and the live
slots of the remainder ring must agree bit for bit, including the chunk that starts inside a group,
completes it and ends inside a later group (its first group reads ring slots
its tail rewrites), and short chunks of several sequences that end inside one
workgroup."""
import numpy as np
import pytest
import torch

from long_context_compressed_append_amd import lcca, synth
from state import State
from gpu_state import GpuState, dev_bytes, dev_typed

pytestmark = pytest.mark.gpu

S = synth.CONFIGS
CASES = [
    synth.shrink(S["csa_64k"], "chunks_csa", (3001, 1024, 500), (120, 70, 90), k=64),
    synth.shrink(S["lp_512k"], "chunks_lp", (2047, 777), (100, 63), k=64),
    synth.shrink(S["prefill_8k"], "chunks_prefill", (3001,), (126,), k=64, win_cap=2048),
    synth.shrink(S["tiny"], "chunks_tiny", (0, 5), (100, 90), win_cap=2048),
    # ten short chunks (66 new tokens): several sequences end inside one
    # 16-token workgroup, each with its own remainder-ring tail
    synth.shrink(S["csa_64k"], "chunks_short", (1001, 1022, 3, 517, 0, 64, 7, 130, 250, 33),
                 (7, 5, 9, 6, 8, 3, 11, 4, 6, 7), k=64),
]


def _tok_rows(arr, dim, rows, tok_f32):
    """Rows of a token array (raw bytes of [n][dim] tokens) as a device tensor."""
    esz = 4 if tok_f32 else 2
    a = arr.reshape(-1).view(np.uint8).reshape(-1, dim * esz)[rows]
    return dev_bytes(a)


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_chunk_and_slice_kernels_store_the_same_bytes(cfg):
    print("compress chunks", cfg.name, flush=True)
    st = State(cfg)
    one = GpuState(st)
    one.compress_append()                          # every chunk in one call
    two = GpuState(st.copy_caches())
    f32 = cfg.tok_dtype == synth.F32
    cu = st.cu_new
    for b in range(cfg.batch):
        n = int(cu[b + 1] - cu[b])
        for lo, hi in ((0, n // 2), (n // 2, n)):
            if hi <= lo:
                continue
            assert hi - lo < 64
            rows = np.arange(cu[b] + lo, cu[b] + hi)
            cnew = np.zeros(cfg.batch + 1, np.int32)
            cnew[b + 1:] = hi - lo
            spos = np.asarray(cfg.prior_len, np.int32).copy()
            spos[b] = cfg.prior_len[b] + lo
            lcca.compress_append(two.pages, dev_typed(cnew), dev_typed(spos), int(hi - lo), two.tok_ldt,
                                 _tok_rows(st.new_kv, cfg.D, rows, f32), dev_typed(st.new_kv_logit[rows]),
                                 _tok_rows(st.new_ik, cfg.dI, rows, f32) if cfg.HI else None,
                                 dev_typed(st.new_ik_logit[rows]) if cfg.HI else None,
                                 two.kv, two.ik, two.win, two.rem)
    torch.cuda.synchronize()
    pairs = [(one.kv.data, two.kv.data), (one.win.data, two.win.data)]
    if one.kv.scale is not None:
        pairs.append((one.kv.scale, two.kv.scale))
    if one.win.scale is not None:
        pairs.append((one.win.scale, two.win.scale))
    if cfg.HI:
        pairs.append((one.ik.data, two.ik.data))
    for i, (a, b) in enumerate(pairs):
        a, b = a.cpu().numpy().view(np.uint8), b.cpu().numpy().view(np.uint8)
        assert np.array_equal(a, b), "array %d differs in %d bytes" % (i, int((a != b).sum()))
    # remainder ring: the live slots, those of each sequence's incomplete last
    # group (the others hold whatever earlier calls left there)
    esz = 4 if f32 else 2
    for what, dim in (("kv", cfg.D), ("ik", cfg.dI)):
        if what == "ik" and not cfg.HI:
            continue
        ra = getattr(one.rem, what).cpu().numpy().view(np.uint8).reshape(cfg.batch, cfg.m, dim * esz)
        rb = getattr(two.rem, what).cpu().numpy().view(np.uint8).reshape(cfg.batch, cfg.m, dim * esz)
        la = getattr(one.rem, what + "_logit").cpu().numpy().reshape(cfg.batch, cfg.m)
        lb = getattr(two.rem, what + "_logit").cpu().numpy().reshape(cfg.batch, cfg.m)
        for b in range(cfg.batch):
            end = cfg.total_len(b)
            for pos in range(end // cfg.m * cfg.m, end):
                assert np.array_equal(ra[b, pos % cfg.m], rb[b, pos % cfg.m]), (what, b, pos)
                assert la[b, pos % cfg.m] == lb[b, pos % cfg.m], (what, b, pos)
