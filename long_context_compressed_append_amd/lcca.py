"""ctypes binding of liblcca.so (declared in include/lcca.h).

Argument marshalling only: torch tensors supply device pointers, the current
torch stream supplies the hipStream_t, and every computation runs in the
library's gfx950 kernels.  There is no fallback: if the library cannot be
loaded, every call raises.

use_debug_library(True) (or LCCA_DEBUG_LIBRARY=1 in the environment) routes
every following call to liblcca_debug.so, whose kernels check the indices
they read from device memory; debug_check() then reports what they found.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

F32, BF16, FP8_E4M3, MXFP4 = 0, 1, 2, 3
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_DEVICE_INDEX = 0, -1, -2, -3, -4, -5
DBG_BLOCK, DBG_ROW, DBG_CHUNK = 1, 2, 4
Q_FP8 = 0x100          # q_dtype flag: FP8 queries on the FP8 matrix cores (lcca.h, LCCA_Q_FP8)
P_BF16 = 0x200         # q_dtype flag of the attention: softmax weights as bf16 alone (lcca.h, LCCA_P_BF16)
ROPE_HALF, ROPE_INVERSE = 1, 2

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblcca.so")
DEBUG_LIB_PATH = os.path.join(_PKG, "liblcca_debug.so")

EXPORTED = ("lcca_compress_append", "lcca_index_logits", "lcca_topk_select", "lcca_sparse_attn_fwd",
            "lcca_sparse_attn_workspace_size", "lcca_topk_workspace_size", "lcca_status_string", "lcca_last_error",
            "lcca_version", "lcca_decode_select", "lcca_decode_select_workspace_size", "lcca_remainder_bytes",
            "lcca_sparse_attn_fwd_noalloc", "lcca_debug_check", "lcca_compress_append_gated", "lcca_rope")


class LccaError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__("lcca status %d: %s" % (status, detail))
        self.status = status


class _Pages(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32), ("block_table", ctypes.c_void_p)]


class _Rows(ctypes.Structure):
    _fields_ = [("num_rows", ctypes.c_int32), ("max_pos", ctypes.c_int32), ("row_seq", ctypes.c_void_p),
                ("row_pos", ctypes.c_void_p)]


class _PagedCache(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("dim", ctypes.c_int32), ("ratio_m", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("data", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class _WindowCache(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("dim", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("window", ctypes.c_int32), ("data", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class _Remainder(ctypes.Structure):
    _fields_ = [("tok_dtype", ctypes.c_int32), ("kv", ctypes.c_void_p), ("ik", ctypes.c_void_p),
                ("kv_logit", ctypes.c_void_p), ("ik_logit", ctypes.c_void_p)]


_LIBS = {}
_USE_DEBUG = os.environ.get("LCCA_DEBUG_LIBRARY") == "1"


def use_debug_library(on: bool = True):
    """Route the calls that follow to liblcca_debug.so (on) or liblcca.so."""
    global _USE_DEBUG
    _USE_DEBUG = bool(on)


def lib():
    """The library in use (built in-tree; compiled first only if absent)."""
    path = DEBUG_LIB_PATH if _USE_DEBUG else LIB_PATH
    L = _LIBS.get(path)
    if L is None:
        if not os.path.exists(path):
            from . import build as _b
            _b.build_one(_USE_DEBUG)
        L = ctypes.CDLL(path)
        P, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        PP, PR, PC, PW, PM = (ctypes.POINTER(_Pages), ctypes.POINTER(_Rows), ctypes.POINTER(_PagedCache),
                              ctypes.POINTER(_WindowCache), ctypes.POINTER(_Remainder))
        L.lcca_compress_append.argtypes = [P, PP, P, P, i32, i32, P, P, P, P, PC, PC, PW, PM]
        L.lcca_compress_append_gated.argtypes = L.lcca_compress_append.argtypes
        L.lcca_index_logits.argtypes = [P, PP, PR, i32, P, i32, P, f32, PC, P, i64]
        L.lcca_topk_select.argtypes = [P, PR, i32, P, i64, i32, P, P, sz]
        L.lcca_sparse_attn_fwd.argtypes = [P, PP, PR, i32, P, i32, i32, f32, PC, P, i32, PW, i32, P, P, P, sz]
        L.lcca_sparse_attn_fwd_noalloc.argtypes = [P, PP, PR, i32, P, i32, i32, f32, PC, P, i32, PW, i32, P, P]
        L.lcca_decode_select.argtypes = [P, PP, PR, P, P, i32, i32, P, P, P, P, PC, PC, PW, PM,
                                         i32, P, i32, P, f32, P, i64, i32, P, P, sz]
        L.lcca_sparse_attn_workspace_size.argtypes = [PR, i32, i32, i32, i32, i32, i32, i32]
        L.lcca_sparse_attn_workspace_size.restype = sz
        L.lcca_topk_workspace_size.argtypes = [PR, i32, i32]
        L.lcca_topk_workspace_size.restype = sz
        L.lcca_decode_select_workspace_size.argtypes = [PR, i32, i32]
        L.lcca_decode_select_workspace_size.restype = sz
        L.lcca_remainder_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.lcca_remainder_bytes.restype = sz
        for n in ("lcca_compress_append", "lcca_index_logits", "lcca_topk_select", "lcca_sparse_attn_fwd",
                  "lcca_decode_select", "lcca_sparse_attn_fwd_noalloc", "lcca_compress_append_gated"):
            getattr(L, n).restype = i32
        L.lcca_debug_check.argtypes = [P, ctypes.POINTER(ctypes.c_uint32)]
        L.lcca_rope.argtypes = [P, i32, P, i64, i32, i32, i32, i32, P, ctypes.c_double, P, i32]
        L.lcca_rope.restype = i32
        L.lcca_debug_check.restype = i32
        L.lcca_status_string.argtypes = [i32]
        for n in ("lcca_status_string", "lcca_last_error", "lcca_version"):
            getattr(L, n).restype = ctypes.c_char_p
        _LIBS[path] = L
    return L


def debug_check(stream=None) -> int:
    """Wait for the stream, then read and clear the debug library's device
    error word: 0 if its kernels found no index out of range, else the
    DBG_* bits of what they found.  Raises on the release library."""
    bits = ctypes.c_uint32(0)
    status = lib().lcca_debug_check(_stream(stream), ctypes.byref(bits))
    if status not in (OK, ERR_DEVICE_INDEX):
        _check(status)
    return int(bits.value)


def version():
    return lib().lcca_version().decode()


def _check(status):
    if status != OK:
        raise LccaError(status, lib().lcca_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    assert t.is_contiguous(), "lcca tensors must be contiguous"
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


# --------------------------------------------------------------------------
# descriptors
# --------------------------------------------------------------------------

@dataclass
class Pages:
    block_table: torch.Tensor            # int32 [batch][max_blocks_per_seq]

    def c(self):
        b, mb = self.block_table.shape
        return _Pages(b, mb, _ptr(self.block_table))


@dataclass
class Rows:
    row_seq: torch.Tensor                # int32 [num_rows]
    row_pos: torch.Tensor                # int32 [num_rows]
    max_pos: int                         # host upper bound of row_pos

    def c(self):
        return _Rows(self.row_seq.numel(), int(self.max_pos), _ptr(self.row_seq), _ptr(self.row_pos))


@dataclass
class PagedCache:
    dtype: int
    dim: int
    ratio_m: int
    num_blocks: int
    data: torch.Tensor                   # uint8 [num_blocks * E * row_bytes]
    scale: Optional[torch.Tensor] = None

    def c(self):
        return _PagedCache(self.dtype, self.dim, self.ratio_m, self.num_blocks, _ptr(self.data), _ptr(self.scale))


@dataclass
class WindowCache:
    dtype: int
    dim: int
    capacity: int
    window: int
    data: torch.Tensor                   # uint8 [batch * capacity * row_bytes]
    scale: Optional[torch.Tensor] = None # float32 [batch * capacity] (FP8)

    def c(self):
        return _WindowCache(self.dtype, self.dim, self.capacity, self.window, _ptr(self.data), _ptr(self.scale))


@dataclass
class Remainder:
    tok_dtype: int
    kv: torch.Tensor
    kv_logit: torch.Tensor
    ik: Optional[torch.Tensor] = None
    ik_logit: Optional[torch.Tensor] = None

    def c(self):
        return _Remainder(self.tok_dtype, _ptr(self.kv), _ptr(self.ik), _ptr(self.kv_logit), _ptr(self.ik_logit))


def remainder_bytes(batch: int, ratio_m: int, kv_dim: int, ik_dim: int, tok_dtype: int) -> int:
    return lib().lcca_remainder_bytes(batch, ratio_m, kv_dim, ik_dim, tok_dtype)


def remainder_in(buf: torch.Tensor, batch: int, ratio_m: int, kv_dim: int, ik_dim: int, tok_dtype: int) -> Remainder:
    """A Remainder whose four arrays are views of one uint8 buffer of
    remainder_bytes() bytes, at the offsets include/lcca.h states."""
    need = remainder_bytes(batch, ratio_m, kv_dim, ik_dim, tok_dtype)
    if need == 0 or buf.numel() * buf.element_size() < need:
        raise LccaError(ERR_INVALID_ARG, "remainder buffer of %d bytes (need %d)" % (buf.numel(), need))
    esz = 4 if tok_dtype == F32 else 2
    slots = batch * ratio_m
    up = lambda x: (x + 255) // 256 * 256
    o_ik = up(slots * kv_dim * esz)
    o_kl = o_ik + up(slots * ik_dim * esz)
    o_il = o_kl + up(slots * 4)
    kv = buf[:slots * kv_dim * esz]
    ik = buf[o_ik:o_ik + slots * ik_dim * esz] if ik_dim else None
    kl = buf[o_kl:o_kl + slots * 4].view(torch.float32)
    il = buf[o_il:o_il + slots * 4].view(torch.float32) if ik_dim else None
    return Remainder(tok_dtype, kv, kl, ik, il)


def _ref(x):
    return ctypes.byref(x) if x is not None else None


# --------------------------------------------------------------------------
# the calls
# --------------------------------------------------------------------------

def compress_append(pages: Pages, cu_new, start_pos, total_new: int, tok_dtype: int, kv_tok, kv_logit,
                    ik_tok, ik_logit, kv: PagedCache, ik: Optional[PagedCache], win: Optional[WindowCache],
                    rem: Remainder, stream=None):
    _check(lib().lcca_compress_append(
        _stream(stream), ctypes.byref(pages.c()), _ptr(cu_new), _ptr(start_pos), int(total_new), tok_dtype,
        _ptr(kv_tok), _ptr(kv_logit), _ptr(ik_tok), _ptr(ik_logit), ctypes.byref(kv.c()),
        _ref(ik.c() if ik else None), _ref(win.c() if win else None), ctypes.byref(rem.c())))


def compress_append_gated(pages: Pages, cu_new, start_pos, total_new: int, tok_dtype: int, kv_tok, kv_logit,
                          ik_tok, ik_logit, kv: PagedCache, ik: Optional[PagedCache], win: Optional[WindowCache],
                          rem: Remainder, stream=None):
    """compress_append with per-channel logits ([n][dim] per stream; the
    remainder ring's logits are [batch][ratio_m][dim])."""
    _check(lib().lcca_compress_append_gated(
        _stream(stream), ctypes.byref(pages.c()), _ptr(cu_new), _ptr(start_pos), int(total_new), tok_dtype,
        _ptr(kv_tok), _ptr(kv_logit), _ptr(ik_tok), _ptr(ik_logit), ctypes.byref(kv.c()),
        _ref(ik.c() if ik else None), _ref(win.c() if win else None), ctypes.byref(rem.c())))


def index_logits(pages: Pages, rows: Rows, q_dtype: int, q_idx, HI: int, w_idx, s_I: float, ik: PagedCache,
                 logits, ld: int, stream=None):
    _check(lib().lcca_index_logits(_stream(stream), ctypes.byref(pages.c()), ctypes.byref(rows.c()), q_dtype,
                                   _ptr(q_idx), HI, _ptr(w_idx), float(s_I), ctypes.byref(ik.c()), _ptr(logits),
                                   int(ld)))


def topk_workspace_size(rows: Rows, ratio_m: int, k: int) -> int:
    return lib().lcca_topk_workspace_size(ctypes.byref(rows.c()), ratio_m, k)


def topk_select(rows: Rows, ratio_m: int, logits, ld: int, k: int, topk_idx, ws=None, stream=None):
    _check(lib().lcca_topk_select(_stream(stream), ctypes.byref(rows.c()), ratio_m, _ptr(logits), int(ld), k,
                                  _ptr(topk_idx), _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0))


def decode_select_workspace_size(rows: Rows, ratio_m: int, k: int) -> int:
    """Bytes of decode_select's workspace; allocate it zeroed (torch.zeros)
    once and reuse it: every call leaves its counts zero."""
    return lib().lcca_decode_select_workspace_size(ctypes.byref(rows.c()), ratio_m, k)


def decode_select(pages: Pages, rows: Rows, cu_new, start_pos, total_new: int, tok_dtype: int, kv_tok, kv_logit,
                  ik_tok, ik_logit, kv: PagedCache, ik: PagedCache, win: Optional[WindowCache], rem: Remainder,
                  q_dtype: int, q_idx, HI: int, w_idx, s_I: float, logits, ld: int, k: int, topk_idx, ws=None,
                  stream=None):
    """compress_append + index_logits + topk_select of a decode step (one new
    token and one row per sequence) with one launch fewer."""
    _check(lib().lcca_decode_select(
        _stream(stream), ctypes.byref(pages.c()), ctypes.byref(rows.c()), _ptr(cu_new), _ptr(start_pos),
        int(total_new), tok_dtype, _ptr(kv_tok), _ptr(kv_logit), _ptr(ik_tok), _ptr(ik_logit), ctypes.byref(kv.c()),
        ctypes.byref(ik.c()), _ref(win.c() if win else None), ctypes.byref(rem.c()), q_dtype, _ptr(q_idx), HI,
        _ptr(w_idx), float(s_I), _ptr(logits), int(ld), k, _ptr(topk_idx), _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0))


def sparse_attn_workspace_size(rows: Rows, ratio_m: int, H: int, dim: int, d_v: int, k: int, topk_given: bool,
                               window: int) -> int:
    return lib().lcca_sparse_attn_workspace_size(ctypes.byref(rows.c()), ratio_m, H, dim, d_v, k,
                                                 1 if topk_given else 0, window)


def sparse_attn_fwd(pages: Pages, rows: Rows, q_dtype: int, q, H: int, d_v: int, sm_scale: float, kv: PagedCache,
                    topk_idx, k: int, win: WindowCache, out_dtype: int, out, lse=None, ws=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().lcca_sparse_attn_fwd(_stream(stream), ctypes.byref(pages.c()), ctypes.byref(rows.c()), q_dtype,
                                      _ptr(q), H, d_v, float(sm_scale), ctypes.byref(kv.c()), _ptr(topk_idx), k,
                                      ctypes.byref(win.c()), out_dtype, _ptr(out), _ptr(lse), _ptr(ws), ws_bytes))


def sparse_attn_fwd_noalloc(pages: Pages, rows: Rows, q_dtype: int, q, H: int, d_v: int, sm_scale: float,
                            kv: PagedCache, topk_idx, k: int, win: WindowCache, out_dtype: int, out, lse=None,
                            stream=None):
    """sparse_attn_fwd with the split partial states in the library's own
    device scratch array (no workspace, no allocation)."""
    _check(lib().lcca_sparse_attn_fwd_noalloc(_stream(stream), ctypes.byref(pages.c()), ctypes.byref(rows.c()),
                                              q_dtype, _ptr(q), H, d_v, float(sm_scale), ctypes.byref(kv.c()),
                                              _ptr(topk_idx), k, ctypes.byref(win.c()), out_dtype, _ptr(out),
                                              _ptr(lse)))


def rope(x, pos, rope_off: int, rope_dim: int, theta: float = 10000.0, inv_freq=None, half: bool = False,
         inverse: bool = False, stream=None):
    """Rotary embedding of dims [rope_off, rope_off + rope_dim) of x
    ([rows][heads][dim], float32 or bfloat16, on the device) in place; row r
    rotated by pos[r] (int32 device).  inv_freq: host float32 [rope_dim / 2]
    or None for theta^(-2i/rope_dim); half: pairs (i, i + rope_dim/2)
    instead of (2i, 2i+1); inverse: rotate back."""
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(x.dtype, -1)
    rows, heads, dim = x.shape
    fr = None
    if inv_freq is not None:
        fr = np.ascontiguousarray(np.asarray(inv_freq, dtype=np.float32))
    flags = (ROPE_HALF if half else 0) | (ROPE_INVERSE if inverse else 0)
    _check(lib().lcca_rope(_stream(stream), dt, _ptr(x), rows, heads, dim, int(rope_off), int(rope_dim), _ptr(pos),
                           float(theta), fr.ctypes.data if fr is not None else None, flags))
