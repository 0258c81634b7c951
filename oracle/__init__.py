"""CPU oracle for compressed-KV attention -- TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 implementation of the four stages (compress+append,
indexer logits, top-k selection, sparse attention with a sliding window),
written in C (``oracle.c``) and wrapped here with ctypes over numpy arrays.
It shares no code with the HIP library and must only be used by the tests,
the smoke check and the CPU-baseline leg of the benchmark.

Byte layouts of the stored caches are the ones the device library uses:

* dtype ``F32`` / ``BF16``: row-major elements.
* dtype ``FP8``: OCP E4M3 codes; an optional float32 scale per row.
* dtype ``MXFP4``: two E2M1 codes per byte (element 2i in the low nibble)
  plus one E8M0 scale byte per 32 elements, in a separate array.

Paged pools are ``[num_blocks][256 // m][row]``; the window ring is
``[batch][capacity][row]``; the remainder ring is ``[batch][m][dim]`` in the
token dtype with float32 logits ``[batch][m]``.
"""
import ctypes
import os

import numpy as np

F32, BF16, FP8, MXFP4 = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib():
    """Load oracle/liboracle.so, compiling it first only if it is absent."""
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.orc_compress_append.argtypes = [i32, i32, P, P, P, i32, P, P, P, P, i32, i32, i32,
                                          i32, P, P, i32, P, P, i32, i32, P, P, P, P, P, P]
        L.orc_compress_append_gated.argtypes = L.orc_compress_append.argtypes
        L.orc_index_logits.argtypes = [i32, P, P, i32, i32, P, i32, P, i32, i32, P, dbl, i32, P, P, P, i64]
        L.orc_topk.argtypes = [i32, P, i32, P, i64, i32, P]
        L.orc_sparse_attn.argtypes = [i32, P, P, i32, i32, P, i32, P, i32, i32, i32, dbl,
                                      i32, P, P, P, i32, i32, i32, i32, P, P, P, P]
        for name in ("orc_compress_append", "orc_compress_append_gated", "orc_index_logits", "orc_topk",
                     "orc_sparse_attn"):
            getattr(L, name).restype = ctypes.c_int
        L.orc_group_compress.argtypes = [i32, i32, P, P, P]
        L.orc_group_compress_gated.argtypes = [i32, i32, P, P, P]
        L.orc_store_rows.argtypes = [i32, P, P, i64, i64, i32, P]
        L.orc_load_rows.argtypes = [i32, P, P, i64, i64, i32, P]
        L.orc_quantize_fp8_rows.argtypes = [P, i64, i32, P, P]
        L.orc_rope.argtypes = [P, i64, i32, i32, i32, i32, P, dbl, P, i32, i32]
        L.orc_mx_scale_exp.argtypes = [ctypes.c_float]
        L.orc_mx_scale_exp.restype = ctypes.c_int
        for name in ("orc_bf16_encode_array", "orc_bf16_decode_array", "orc_fp8_encode_array",
                     "orc_fp8_decode_array", "orc_fp4_encode_array", "orc_fp4_decode_array"):
            getattr(L, name).argtypes = [P, i64, P]
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_set_num_threads.argtypes = [i32]
        _LIB = L
    return _LIB


def _p(a):
    """Raw pointer of a C-contiguous numpy array (or NULL for None)."""
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def row_bytes(dtype, dim):
    return {F32: 4 * dim, BF16: 2 * dim, FP8: dim, MXFP4: dim // 2}[dtype]


def num_threads():
    return lib().orc_num_threads()


def set_num_threads(n):
    """Threads of the oracle's parallel loops from now on."""
    lib().orc_set_num_threads(int(n))


# --------------------------------------------------------------------------
# codecs (element-wise)
# --------------------------------------------------------------------------

def bf16_encode(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_bf16_encode_array(_p(x), x.size, _p(out))
    return out


def bf16_decode(h):
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().orc_bf16_decode_array(_p(h), h.size, _p(out))
    return out


def fp8_encode(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().orc_fp8_encode_array(_p(x), x.size, _p(out))
    return out


def rope(x, pos, off, rd, theta=10000.0, freq=None, pairing=0, inverse=False):
    """Rotary embedding of dims [off, off + rd) of x [rows][heads][dim] (fp64
    copy returned), row r rotated by pos[r]; pairing 0: pairs (2i, 2i+1),
    1: (i, i + rd/2); freq: float32 [rd/2] or None for theta^(-2i/rd)."""
    y = np.array(x, dtype=np.float64, order="C", copy=True)
    rows, heads, dim = y.shape
    fr = None if freq is None else np.ascontiguousarray(freq, dtype=np.float32)
    lib().orc_rope(_p(y), rows, heads, dim, off, rd, _p(_i32(pos)), float(theta), None if fr is None else _p(fr),
                   int(pairing), int(bool(inverse)))
    return y


def quantize_fp8_rows(x):
    """FP8 rows with a power-of-two scale: x [n][dim] float32 -> (codes uint8
    [n][dim], X int32 [n]); x ~ decode(codes) * 2^X."""
    x = np.ascontiguousarray(x, np.float32)
    n, dim = x.shape
    codes = np.empty((n, dim), np.uint8)
    X = np.empty(n, np.int32)
    lib().orc_quantize_fp8_rows(_p(x), n, dim, _p(codes), _p(X))
    return codes, X


def fp8_decode(c):
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().orc_fp8_decode_array(_p(c), c.size, _p(out))
    return out


def fp4_encode(v):
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint8)
    lib().orc_fp4_encode_array(_p(v), v.size, _p(out))
    return out


def fp4_decode(c):
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().orc_fp4_decode_array(_p(c), c.size, _p(out))
    return out


def mx_scale_exp(amax):
    return lib().orc_mx_scale_exp(ctypes.c_float(float(amax)))


# --------------------------------------------------------------------------
# stored rows
# --------------------------------------------------------------------------

def alloc_rows(dtype, nrows, dim, with_scale):
    """Zeroed storage for nrows rows: (data uint8, scale or None)."""
    data = np.zeros(nrows * row_bytes(dtype, dim), np.uint8)
    scale = None
    if dtype == MXFP4:
        scale = np.zeros(nrows * (dim // 32), np.uint8)
    elif dtype == FP8 and with_scale:
        scale = np.ones(nrows, np.float32)
    return data, scale


def store_rows(dtype, data, scale, first_row, x):
    """Encode float32 rows x [n][dim] into rows first_row.. of (data, scale)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    n, dim = x.shape
    assert data.nbytes >= (first_row + n) * row_bytes(dtype, dim)
    lib().orc_store_rows(dtype, _p(data), _p(scale), first_row, n, dim, _p(x))


def load_rows(dtype, data, scale, first_row, n, dim):
    """Dequantise stored rows into float64 [n][dim]."""
    assert data.nbytes >= (first_row + n) * row_bytes(dtype, dim)
    out = np.empty((n, dim), np.float64)
    lib().orc_load_rows(dtype, _p(data), _p(scale), first_row, n, dim, _p(out))
    return out


def group_compress(x, a):
    """Softmax-weighted aggregation of one group: x [m][dim], a [m] -> C [dim] (fp64)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    a = np.ascontiguousarray(a, dtype=np.float64)
    m, dim = x.shape
    C = np.empty(dim, np.float64)
    lib().orc_group_compress(m, dim, _p(x), _p(a), _p(C))
    return C


def group_compress_gated(x, a):
    """Per-channel-gated aggregation of one group: x [m][dim], a [m][dim] -> C [dim] (fp64)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    a = np.ascontiguousarray(a, dtype=np.float64)
    m, dim = x.shape
    assert a.shape == (m, dim)
    C = np.empty(dim, np.float64)
    lib().orc_group_compress_gated(m, dim, _p(x), _p(a), _p(C))
    return C


# --------------------------------------------------------------------------
# the four stages (arrays are numpy; caches are mutated in place)
# --------------------------------------------------------------------------

def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def compress_append(block_table, cu_new, start_pos, tok_dtype, kv_tok, kv_logit, ik_tok, ik_logit,
                    m, D, dI, kv, ik, win, rem, gated=False):
    """kv/ik: dict(dtype, data, scale); win: dict(dtype, cap, data, scale) or None;
    rem: dict(kv, ik, kv_logit, ik_logit).  Token arrays hold raw bytes of the
    token dtype (float32 or bf16 bit patterns as uint16).  gated: the
    per-channel-gated variant (logits [n][dim], ring logits [batch][m][dim])."""
    bt = _i32(block_table)
    batch, max_blocks = bt.shape
    cu = _i32(cu_new)
    sp = _i32(start_pos)
    has_ik = ik is not None and ik_tok is not None
    fn = lib().orc_compress_append_gated if gated else lib().orc_compress_append
    rc = fn(
        batch, max_blocks, _p(bt), _p(cu), _p(sp),
        tok_dtype, _p(kv_tok), _p(np.ascontiguousarray(kv_logit, np.float32)),
        _p(ik_tok) if has_ik else None,
        _p(np.ascontiguousarray(ik_logit, np.float32)) if has_ik else None,
        m, D, dI if has_ik else 0,
        kv["dtype"], _p(kv["data"]), _p(kv["scale"]),
        ik["dtype"] if has_ik else 0, _p(ik["data"]) if has_ik else None, _p(ik["scale"]) if has_ik else None,
        win["dtype"] if win else 0, win["cap"] if win else 1, _p(win["data"]) if win else None,
        _p(win["scale"]) if win else None,
        _p(rem["kv"]), _p(rem["ik"]) if has_ik else None, _p(rem["kv_logit"]),
        _p(rem["ik_logit"]) if has_ik else None)
    assert rc == 0


def index_logits(row_seq, row_pos, m, block_table, q_dtype, q_idx, HI, dI, w_idx, s_I, ik, ld):
    rs, rp, bt = _i32(row_seq), _i32(row_pos), _i32(block_table)
    rows = rs.shape[0]
    out = np.zeros((rows, ld), np.float64)
    rc = lib().orc_index_logits(rows, _p(rs), _p(rp), m, bt.shape[1], _p(bt), q_dtype,
                                _p(np.ascontiguousarray(q_idx)), HI, dI,
                                _p(np.ascontiguousarray(w_idx, np.float32)), float(s_I),
                                ik["dtype"], _p(ik["data"]), _p(ik["scale"]), _p(out), ld)
    assert rc == 0
    return out


def topk(row_pos, m, logits, k):
    rp = _i32(row_pos)
    lg = np.ascontiguousarray(logits, dtype=np.float64)
    rows, ld = lg.shape
    idx = np.empty((rows, k), np.int32)
    rc = lib().orc_topk(rows, _p(rp), m, _p(lg), ld, k, _p(idx))
    assert rc == 0
    return idx


def sparse_attn(row_seq, row_pos, m, block_table, q_dtype, q, H, D, d_v, sm_scale, kv,
                topk_idx, k, win, window):
    rs, rp, bt = _i32(row_seq), _i32(row_pos), _i32(block_table)
    rows = rs.shape[0]
    out = np.zeros((rows, H, d_v), np.float64)
    lse = np.zeros((rows, H), np.float64)
    ti = _i32(topk_idx) if topk_idx is not None else None
    rc = lib().orc_sparse_attn(rows, _p(rs), _p(rp), m, bt.shape[1], _p(bt), q_dtype,
                               _p(np.ascontiguousarray(q)), H, D, d_v, float(sm_scale),
                               kv["dtype"], _p(kv["data"]), _p(kv["scale"]), _p(ti), k,
                               win["dtype"] if win else 0, win["cap"] if win else 1, window,
                               _p(win["data"]) if win else None, _p(win["scale"]) if win else None,
                               _p(out), _p(lse))
    assert rc == 0
    return out, lse
