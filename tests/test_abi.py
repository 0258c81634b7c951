"""The C ABI: the library loads, exports every function include/lcca.h
declares, and rejects invalid arguments on the host before any launch
(these calls return before touching the GPU, so they run anywhere)."""
import ctypes
import os
import re

import pytest

from long_context_compressed_append_amd import lcca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "lcca.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lcca_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = lcca.lib()
    names = _declared()
    assert set(names) == set(lcca.EXPORTED)
    for n in names:
        assert hasattr(L, n), n
    assert "gfx950" in lcca.version()


def test_status_strings():
    L = lcca.lib()
    for s in (0, -1, -2, -3, -4, -5):
        assert L.lcca_status_string(s) != b"unknown status"


def test_debug_library_exports_the_same_symbols():
    import ctypes as C
    D = C.CDLL(lcca.DEBUG_LIB_PATH)
    for n in _declared():
        assert hasattr(D, n), n
    D.lcca_version.restype = C.c_char_p
    assert b"LCCA_DEBUG" in D.lcca_version()
    assert b"LCCA_DEBUG" not in lcca.lib().lcca_version()


def test_release_library_has_no_debug_word():
    bits = ctypes.c_uint32(7)
    assert lcca.lib().lcca_debug_check(None, ctypes.byref(bits)) == lcca.ERR_UNSUPPORTED
    assert bits.value == 0
    assert b"LCCA_DEBUG" in lcca.lib().lcca_last_error()
    with pytest.raises(lcca.LccaError):
        lcca.debug_check(0)                  # the null stream: nothing runs on it


def _pool(dtype=lcca.BF16, dim=576, m=4, blocks=4, data=1):
    return lcca._PagedCache(dtype, dim, m, blocks, data, None)


def test_invalid_arguments_rejected_before_launch():
    L = lcca.lib()
    pages = lcca._Pages(1, 4, 1)
    rows = lcca._Rows(1, 100, 1, 1)
    ik = _pool(lcca.BF16, 128)
    by = ctypes.byref
    # NULL pages
    assert L.lcca_index_logits(None, None, by(rows), lcca.BF16, 1, 64, 1, 1.0, by(ik), 1, 64) == lcca.ERR_INVALID_ARG
    assert b"pages" in L.lcca_last_error()
    # ld too small for the visible entries
    assert L.lcca_index_logits(None, by(pages), by(rows), lcca.BF16, 1, 64, 1, 1.0, by(ik), 1, 10) == lcca.ERR_INVALID_ARG
    # unsupported head count for the MFMA path
    assert L.lcca_index_logits(None, by(pages), by(rows), lcca.BF16, 1, 48, 1, 1.0, by(ik), 1, 64) == lcca.ERR_UNSUPPORTED
    # max_pos beyond the block table
    far = lcca._Rows(1, 4 * 256, 1, 1)
    assert L.lcca_index_logits(None, by(pages), by(far), lcca.BF16, 1, 64, 1, 1.0, by(ik), 1, 4096) == lcca.ERR_INVALID_ARG
    # bad ratio
    bad = _pool(lcca.BF16, 128, m=3)
    assert L.lcca_index_logits(None, by(pages), by(rows), lcca.BF16, 1, 64, 1, 1.0, by(bad), 1, 64) == lcca.ERR_INVALID_ARG
    # top-k: k < 1
    assert L.lcca_topk_select(None, by(rows), 4, 1, 64, 0, 1, None, 0) == lcca.ERR_INVALID_ARG
    # top-k: more visible entries than the selection's row bitmaps hold (2^18)
    huge = lcca._Rows(1, 4 * (1 << 18) + 3, 1, 1)
    assert L.lcca_topk_select(None, by(huge), 4, 1, (1 << 18) + 1, 64, 1, None, 0) == lcca.ERR_UNSUPPORTED
    # rows of more than 32768 entries need the two-launch workspace
    long_rows = lcca._Rows(3, 4 * 40000 - 1, 1, 1)
    need = L.lcca_topk_workspace_size(by(long_rows), 4, 2048)
    assert need == 3 * (3 * 2048) * 8            # 3 slices of 16384, k candidates each, key + entry
    assert L.lcca_topk_workspace_size(by(rows), 4, 64) == 0
    assert L.lcca_topk_select(None, by(long_rows), 4, 1, 40000, 2048, 1, None, 0) == lcca.ERR_WORKSPACE
    assert b"workspace" in L.lcca_last_error()
    ok = lcca._Rows(1, 4 * (1 << 18) - 1, 1, 1)
    assert L.lcca_topk_select(None, by(ok), 4, 1, 1 << 18, 0, 1, None, 0) == lcca.ERR_INVALID_ARG   # k < 1 only
    # long rows whose slices' candidates (16 slices x k) exceed the 2^18 bits of
    # the candidates' selection bitmaps, with an ample workspace
    need = L.lcca_topk_workspace_size(by(ok), 4, 16385)
    assert L.lcca_topk_select(None, by(ok), 4, 1, 1 << 18, 16385, 1, 16, need) == lcca.ERR_UNSUPPORTED
    assert b"candidates" in L.lcca_last_error()
    # at the limit (16 x 16384 = 2^18) the call gets past validation; the
    # misaligned workspace pointer then stops it before any launch
    need = L.lcca_topk_workspace_size(by(ok), 4, 16384)
    assert L.lcca_topk_select(None, by(ok), 4, 1, 1 << 18, 16384, 1, 8, need) == lcca.ERR_INVALID_ARG
    assert b"aligned" in L.lcca_last_error()
    # attention: workspace too small (16 rows of 64K context need key splits)
    kv = _pool(lcca.BF16, 576, blocks=4096)
    win = lcca._WindowCache(lcca.FP8_E4M3, 576, 128, 128, 1, 1)
    pg = lcca._Pages(16, 256, 1)
    rw = lcca._Rows(16, 65535, 1, 1)
    need = L.lcca_sparse_attn_workspace_size(by(rw), 4, 64, 576, 576, 2048, 1, 128)
    assert need > 0
    st = L.lcca_sparse_attn_fwd(None, by(pg), by(rw), lcca.BF16, 1, 64, 576, 0.04, by(kv), 1, 2048, by(win),
                                lcca.F32, 1, None, 1, need - 1)
    assert st == lcca.ERR_WORKSPACE
    # a large enough workspace that is not 16-byte aligned
    st = L.lcca_sparse_attn_fwd(None, by(pg), by(rw), lcca.BF16, 1, 64, 576, 0.04, by(kv), 1, 2048, by(win),
                                lcca.F32, 1, None, 8, need)
    assert st == lcca.ERR_INVALID_ARG and b"aligned" in L.lcca_last_error()
    # FP8 window without its scale array
    win_ns = lcca._WindowCache(lcca.FP8_E4M3, 576, 128, 128, 1, None)
    st = L.lcca_sparse_attn_fwd(None, by(pg), by(rw), lcca.BF16, 1, 64, 576, 0.04, by(kv), 1, 2048, by(win_ns),
                                lcca.F32, 1, None, 1, need)
    assert st == lcca.ERR_INVALID_ARG
    # MXFP4 indexer pool is not a supported combination
    rem = lcca._Remainder(lcca.BF16, 1, 1, 1, 1)
    mx = _pool(lcca.MXFP4, 128)
    mx.scale = 1
    st = L.lcca_compress_append(None, by(pages), 1, 1, 1, lcca.BF16, 1, 1, 1, 1, by(kv), by(mx), None, by(rem))
    assert st == lcca.ERR_UNSUPPORTED
    # token dtype must match the remainder ring
    rem32 = lcca._Remainder(lcca.F32, 1, 1, 1, 1)
    st = L.lcca_compress_append(None, by(pages), 1, 1, 1, lcca.BF16, 1, 1, 1, 1, by(kv), by(ik), None, by(rem32))
    assert st == lcca.ERR_INVALID_ARG


def test_binding_raises_on_error():
    import torch
    t = torch.zeros(4, dtype=torch.int32)
    rows = lcca.Rows(t, t, 100)
    with pytest.raises(lcca.LccaError) as e:
        lcca.topk_select(rows, 4, t, 10, 64, t, stream=0)
    assert e.value.status == lcca.ERR_INVALID_ARG


def test_empty_calls_return_ok_without_launching():
    """Zero new tokens / zero rows: validated, then nothing is launched (so
    these run without a GPU)."""
    L = lcca.lib()
    by = ctypes.byref
    pages = lcca._Pages(1, 4, 1)
    kv = _pool(lcca.BF16, 576)
    ik = _pool(lcca.BF16, 128)
    win = lcca._WindowCache(lcca.BF16, 576, 128, 128, 1, None)
    rem = lcca._Remainder(lcca.BF16, 1, 1, 1, 1)
    st = L.lcca_compress_append(None, by(pages), 1, 1, 0, lcca.BF16, None, None, None, None, by(kv), by(ik),
                                by(win), by(rem))
    assert st == lcca.OK, L.lcca_last_error()
    none = lcca._Rows(0, 0, 1, 1)
    assert L.lcca_index_logits(None, by(pages), by(none), lcca.BF16, 1, 64, 1, 1.0, by(ik), 1, 64) == lcca.OK
    assert L.lcca_topk_select(None, by(none), 4, 1, 64, 64, 1, None, 0) == lcca.OK
    assert L.lcca_sparse_attn_workspace_size(by(none), 4, 64, 576, 576, 64, 1, 128) == 0
    st = L.lcca_sparse_attn_fwd(None, by(pages), by(none), lcca.BF16, 1, 64, 576, 0.04, by(kv), 1, 64, by(win),
                                lcca.F32, 1, None, None, 0)
    assert st == lcca.OK, L.lcca_last_error()


def test_decode_select_rejects_what_it_does_not_cover():
    """The fused decode call checks its contract and supported shapes on the
    host and launches nothing when they fail."""
    L = lcca.lib()
    by = ctypes.byref
    pages = lcca._Pages(16, 256, 1)
    kv = _pool(lcca.BF16, 576, blocks=4096)
    ik = _pool(lcca.BF16, 128, blocks=4096)
    win = lcca._WindowCache(lcca.FP8_E4M3, 576, 128, 128, 1, 1)
    rem = lcca._Remainder(lcca.BF16, 1, 1, 1, 1)
    rows = lcca._Rows(16, 65535, 1, 1)

    def call(rows=rows, total_new=16, tok=lcca.BF16, ik=ik, rem=rem, ld=16384, pages=pages):
        return L.lcca_decode_select(None, by(pages), by(rows), 1, 1, total_new, tok, 1, 1, 1, 1, by(kv),
                                    by(ik) if ik is not None else None, by(win), by(rem), lcca.BF16, 1, 64, 1, 1.0,
                                    16, ld, 2048, 1, None, 0)

    # one row and one new token per sequence
    assert call(total_new=15) == lcca.ERR_INVALID_ARG
    assert call(rows=lcca._Rows(8, 65535, 1, 1)) == lcca.ERR_INVALID_ARG
    assert b"one new token" in L.lcca_last_error()
    # the indexer pool is required
    assert call(ik=None) == lcca.ERR_INVALID_ARG
    # the workspace of the leading-digit counts: missing, or not 16-byte aligned
    assert call() == lcca.ERR_WORKSPACE
    need = L.lcca_decode_select_workspace_size(by(rows), 4, 2048)
    assert need == 16 * 4096 * 4
    st = L.lcca_decode_select(None, by(pages), by(rows), 1, 1, 16, lcca.BF16, 1, 1, 1, 1, by(kv), by(ik), by(win),
                              by(rem), lcca.BF16, 1, 64, 1, 1.0, 16, 16384, 2048, 1, 8, need)
    assert st == lcca.ERR_INVALID_ARG and b"aligned" in L.lcca_last_error()
    # fp32 tokens, logit rows not 16-byte aligned
    rem32 = lcca._Remainder(lcca.F32, 1, 1, 1, 1)
    assert call(tok=lcca.F32, rem=rem32) == lcca.ERR_UNSUPPORTED
    assert call(ld=16386) == lcca.ERR_UNSUPPORTED
    # rows of more than 32K entries: the slices' workspace is required, and
    # their candidates (slices x k) must fit the compact selection
    big = lcca._Pages(16, 1024, 1)
    assert call(rows=lcca._Rows(16, 4 * 40000 - 1, 1, 1), ld=40000, pages=big) == lcca.ERR_WORKSPACE
    # their workspace: the slices' candidates, then the leading-digit counts
    rows_40k = lcca._Rows(16, 4 * 40000 - 1, 1, 1)
    assert (L.lcca_decode_select_workspace_size(by(rows_40k), 4, 2048)
            == L.lcca_topk_workspace_size(by(rows_40k), 4, 2048) + 16 * 4096 * 4)
    huge = lcca._Pages(16, 4096, 1)
    rows_long = lcca._Rows(16, 4 * 262143 - 1, 1, 1)
    need = L.lcca_topk_workspace_size(by(rows_long), 4, 4096)
    st = L.lcca_decode_select(None, by(huge), by(rows_long), 1, 1, 16, lcca.BF16, 1, 1, 1, 1, by(kv), by(ik), by(win),
                              by(rem), lcca.BF16, 1, 64, 1, 1.0, 16, 262144, 4096, 1, 16, need)
    assert st == lcca.ERR_UNSUPPORTED       # 16 slices x 4096 candidates > 32,768


def test_remainder_bytes_layout():
    """lcca_remainder_bytes: kv, ik, kv_logit, ik_logit carved from one
    buffer, each starting on a 256-byte boundary."""
    L = lcca.lib()
    up = lambda x: (x + 255) // 256 * 256
    # 16 sequences, m = 4, bf16 tokens of 576 + 128 dims
    want = up(16 * 4 * 576 * 2) + up(16 * 4 * 128 * 2) + up(16 * 4 * 4) + 16 * 4 * 4
    assert L.lcca_remainder_bytes(16, 4, 576, 128, lcca.BF16) == want
    # no indexer stream: kv and kv_logit only
    assert L.lcca_remainder_bytes(4, 128, 576, 0, lcca.BF16) == up(4 * 128 * 576 * 2) + 4 * 128 * 4
    # fp32 tokens
    assert L.lcca_remainder_bytes(1, 4, 128, 32, lcca.F32) == up(4 * 128 * 4) + up(4 * 32 * 4) + up(16) + 16
    # invalid arguments: 0
    for args in ((0, 4, 576, 128, lcca.BF16), (1, 3, 576, 128, lcca.BF16), (1, 4, 0, 128, lcca.BF16),
                 (1, 4, 576, -1, lcca.BF16), (1, 4, 576, 128, lcca.FP8_E4M3)):
        assert L.lcca_remainder_bytes(*args) == 0, args
    import torch
    buf = torch.zeros(want, dtype=torch.uint8)
    rem = lcca.remainder_in(buf, 16, 4, 576, 128, lcca.BF16)
    base = buf.data_ptr()
    assert rem.kv.data_ptr() == base
    assert rem.ik.data_ptr() - base == up(16 * 4 * 576 * 2)
    assert rem.kv_logit.data_ptr() - base == up(16 * 4 * 576 * 2) + up(16 * 4 * 128 * 2)
    assert rem.ik_logit.data_ptr() - rem.kv_logit.data_ptr() == up(16 * 4 * 4)
    assert rem.ik_logit.data_ptr() + rem.ik_logit.numel() * 4 - base == want
    with pytest.raises(lcca.LccaError):
        lcca.remainder_in(buf[:want - 1], 16, 4, 576, 128, lcca.BF16)


def test_noalloc_rejects_plans_beyond_its_scratch():
    """lcca_sparse_attn_fwd_noalloc refuses, before any launch, arguments whose
    split partial states exceed its scratch array (64 MiB)."""
    L = lcca.lib()
    by = ctypes.byref
    pages = lcca._Pages(100, 4096, 1)
    rows = lcca._Rows(100, (1 << 20) - 1, 1, 1)
    kv = _pool(lcca.BF16, 576, m=128, blocks=4096 * 100)
    win = lcca._WindowCache(lcca.FP8_E4M3, 576, 128, 128, 1, 1)
    need = L.lcca_sparse_attn_workspace_size(by(rows), 128, 640, 576, 576, 0, 0, 128)
    assert need > (64 << 20)
    st = L.lcca_sparse_attn_fwd_noalloc(None, by(pages), by(rows), lcca.BF16, 1, 640, 576, 0.04, by(kv), None, 0,
                                        by(win), lcca.F32, 1, None)
    assert st == lcca.ERR_UNSUPPORTED and b"scratch" in L.lcca_last_error()
    # the same validation as the workspace entry point
    st = L.lcca_sparse_attn_fwd_noalloc(None, by(pages), by(rows), lcca.BF16, None, 640, 576, 0.04, by(kv), None,
                                        0, by(win), lcca.F32, 1, None)
    assert st == lcca.ERR_INVALID_ARG


def test_rope_arguments_checked_before_launch():
    """lcca_rope rejects what it does not cover on the host (dummy pointers:
    nothing is launched), and zero rows is a no-op."""
    L = lcca.lib()
    R = lambda dt, rows, heads, dim, off, rd, theta=10000.0, fr=None, flags=0: L.lcca_rope(
        None, dt, 16, rows, heads, dim, off, rd, 16, theta, fr, flags)
    assert R(lcca.FP8_E4M3, 4, 2, 64, 0, 64) == lcca.ERR_UNSUPPORTED
    assert R(lcca.MXFP4, 4, 2, 64, 0, 64) == lcca.ERR_UNSUPPORTED
    for args in ((4, 2, 64, 0, 63), (4, 2, 64, 0, 0), (4, 2, 64, 2, 64), (4, 2, 600, 0, 258), (4, 2, 64, -2, 32),
                 (-1, 2, 64, 0, 64), (4, 0, 64, 0, 64), (4, 2, 0, 0, 2)):
        assert R(lcca.F32, *args) == lcca.ERR_INVALID_ARG, args
    assert R(lcca.F32, 4, 2, 64, 0, 64, flags=4) == lcca.ERR_INVALID_ARG
    for th in (0.0, -1.0, float("inf"), float("nan")):
        assert R(lcca.BF16, 4, 2, 64, 0, 64, theta=th) == lcca.ERR_INVALID_ARG, th
    bad = (ctypes.c_float * 32)(*([1.0] * 31 + [float("inf")]))
    assert R(lcca.F32, 4, 2, 64, 0, 64, fr=ctypes.cast(bad, ctypes.c_void_p)) == lcca.ERR_INVALID_ARG
    assert "frequency 31" in lcca.lib().lcca_last_error().decode()
    assert L.lcca_rope(None, lcca.F32, None, 4, 2, 64, 0, 64, None, 1e4, None, 0) == lcca.ERR_INVALID_ARG
    assert L.lcca_rope(None, lcca.F32, None, 0, 2, 64, 0, 64, None, 1e4, None, 0) == lcca.OK
    assert L.lcca_rope(None, lcca.BF16, None, 0, 1, 576, 512, 64, None, 0.0, None, 3) == lcca.ERR_INVALID_ARG
