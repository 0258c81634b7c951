"""Compressed-KV decode and chunked-prefill attention for AMD Instinct MI355X (gfx950).

Four stages behind a C-ABI library (``liblcca.so``, declared in
``include/lcca.h``): compress_append, index_logits, topk_select and
sparse_attn_fwd.  The Python side (``lcca``) only marshals arguments.
"""
__all__ = ["lcca", "synth"]
