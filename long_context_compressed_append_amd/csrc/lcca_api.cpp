// Host side of liblcca: argument validation, launch planning and dispatch of
// the gfx950 kernels.  Every check runs before any launch; a failed check
// returns an error code and launches nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstring>

#include "../../include/lcca.h"
#include "device.h"
#include "kernels.h"

namespace lcca {
int attn_f32_max_keys();
int attn_max_split_tiles();
int attn_max_splits();
int attn_tile_keys();
// the scratch array of lcca_sparse_attn_fwd_noalloc (attn_scratch.hip)
size_t attn_scratch_bytes();
hipError_t attn_scratch(void** ptr);
}

static_assert(lcca::kDbgBlock == LCCA_DBG_BLOCK && lcca::kDbgRow == LCCA_DBG_ROW && lcca::kDbgChunk == LCCA_DBG_CHUNK,
              "device error word bits");

namespace {

thread_local char g_err[512] = "";

lcca_status fail(lcca_status code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

lcca_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return LCCA_OK;
    return fail(LCCA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool valid_m(int m) { return m >= 1 && m <= 256 && 256 % m == 0; }

// Visible entries of a row at position max_pos, without int overflow.
int64_t max_visible(int32_t max_pos, int m) { return ((int64_t)max_pos + 1) / m; }

// Byte counts that saturate at SIZE_MAX (a workspace no caller can provide)
// instead of wrapping.
size_t mul_sat(size_t a, size_t b) {
    size_t r;
    return __builtin_mul_overflow(a, b, &r) ? SIZE_MAX : r;
}
size_t add_sat(size_t a, size_t b) {
    size_t r;
    return __builtin_add_overflow(a, b, &r) ? SIZE_MAX : r;
}
size_t up256(size_t x) { return x > SIZE_MAX - 255 ? SIZE_MAX : (x + 255) & ~(size_t)255; }

// The device error word the kernels of a debug build record index
// violations in (nullptr in release builds).
lcca_status debug_word(uint32_t** w) { return hip_status(lcca::debug_word(w), "debug error word lookup"); }

bool valid_dtype(int d) { return d >= LCCA_F32 && d <= LCCA_MXFP4; }

lcca_status check_pages(const lcca_pages* pg) {
    if (!pg) return fail(LCCA_ERR_INVALID_ARG, "pages is NULL");
    if (pg->batch < 1 || pg->max_blocks_per_seq < 1 || !pg->block_table)
        return fail(LCCA_ERR_INVALID_ARG, "pages: batch=%d max_blocks_per_seq=%d block_table=%p", pg->batch,
                    pg->max_blocks_per_seq, (const void*)pg->block_table);
    return LCCA_OK;
}

lcca_status check_rows(const lcca_rows* rw, int ratio_m, int max_blocks) {
    if (!rw) return fail(LCCA_ERR_INVALID_ARG, "rows is NULL");
    if (rw->num_rows < 0) return fail(LCCA_ERR_INVALID_ARG, "rows: num_rows=%d", rw->num_rows);
    if (rw->num_rows > 0 && (!rw->row_seq || !rw->row_pos))
        return fail(LCCA_ERR_INVALID_ARG, "rows: row_seq/row_pos NULL");
    if (rw->max_pos < 0) return fail(LCCA_ERR_INVALID_ARG, "rows: max_pos=%d", rw->max_pos);
    if (max_blocks > 0 && (int64_t)rw->max_pos >= (int64_t)max_blocks * 256)
        return fail(LCCA_ERR_INVALID_ARG, "rows: max_pos=%d beyond the block table (%d blocks of 256)", rw->max_pos,
                    max_blocks);
    (void)ratio_m;
    return LCCA_OK;
}

lcca_status check_pool(const lcca_paged_cache* c, const char* name) {
    if (!c) return fail(LCCA_ERR_INVALID_ARG, "%s is NULL", name);
    if (!valid_dtype(c->dtype) || c->dim < 1 || !valid_m(c->ratio_m) || c->num_blocks < 1 || !c->data)
        return fail(LCCA_ERR_INVALID_ARG, "%s: dtype=%d dim=%d ratio_m=%d num_blocks=%d data=%p", name, c->dtype,
                    c->dim, c->ratio_m, c->num_blocks, c->data);
    if (c->dtype == LCCA_MXFP4 && (c->dim % 32 != 0 || !c->scale))
        return fail(LCCA_ERR_INVALID_ARG, "%s: MXFP4 needs dim %% 32 == 0 and a scale array", name);
    return LCCA_OK;
}

lcca_status check_window(const lcca_window_cache* w, int dim) {
    if (!w) return fail(LCCA_ERR_INVALID_ARG, "window is NULL");
    if (w->dtype != LCCA_F32 && w->dtype != LCCA_BF16 && w->dtype != LCCA_FP8_E4M3)
        return fail(LCCA_ERR_UNSUPPORTED, "window dtype %d (F32, BF16 or FP8_E4M3)", w->dtype);
    if (w->dim != dim || w->capacity < 1 || w->window < 1 || w->window > w->capacity || !w->data)
        return fail(LCCA_ERR_INVALID_ARG, "window: dim=%d (want %d) capacity=%d window=%d data=%p", w->dim, dim,
                    w->capacity, w->window, w->data);
    if (w->dtype == LCCA_FP8_E4M3 && !w->scale) return fail(LCCA_ERR_INVALID_ARG, "FP8 window needs a scale array");
    return LCCA_OK;
}

struct AttnPlan {
    int nsplit, split_tiles;
    size_t ws_bytes;
};

// Split plan of the bf16 attention kernels.  A row's key list is its
// selected part padded to whole 32-key tiles, then the window tiles.  Rows
// are split into ranges of whole tiles across workgroups only when the rows
// alone cannot fill the 256 compute units (and a split never exceeds the
// kernel's per-split index cache); partial softmax states then go to the
// workspace for the merge kernel.
AttnPlan attn_plan(int rows, int max_pos, int m, int H, int d_v, int k, bool topk_given, int window) {
    AttnPlan p{1, 1, 0};
    if (rows <= 0) return p;
    const int64_t nvis = max_visible(max_pos, m);
    const int64_t nsel = topk_given ? (int64_t)k : nvis;
    const int64_t nwin = std::min<int64_t>(window, (int64_t)max_pos + 1);
    const int64_t key_tiles = lcca::attn_tile_keys();
    const int64_t tiles = std::max<int64_t>(1, (nsel + key_tiles - 1) / key_tiles + (nwin + key_tiles - 1) / key_tiles);
    const int64_t max_tps = lcca::attn_max_split_tiles();
    constexpr int kTargetWorkgroups = 256;
    int64_t tps = rows >= kTargetWorkgroups / 2 ? tiles : (tiles * rows + kTargetWorkgroups - 1) / kTargetWorkgroups;
    tps = std::max<int64_t>(1, std::min<int64_t>(tps, max_tps));
    int64_t nsplit = (tiles + tps - 1) / tps;
    if (nsplit > lcca::attn_max_splits()) {
        tps = (tiles + lcca::attn_max_splits() - 1) / lcca::attn_max_splits();
        nsplit = (tiles + tps - 1) / tps;
    }
    p.nsplit = (int)nsplit;
    p.split_tiles = (int)tps;
    if (p.nsplit > 1) {
        const size_t parts = mul_sat(mul_sat(mul_sat((size_t)rows, (size_t)p.nsplit), (size_t)H), (size_t)d_v);
        const size_t po = up256(mul_sat(parts, sizeof(float)));
        p.ws_bytes = add_sat(po, mul_sat(mul_sat((size_t)rows * p.nsplit, 2 * (size_t)H), sizeof(float)));
    }
    return p;
}

}  // namespace

extern "C" {

const char* lcca_last_error(void) { return g_err; }

size_t lcca_remainder_bytes(int32_t batch, int32_t ratio_m, int32_t kv_dim, int32_t ik_dim, int32_t tok_dtype) {
    if (batch < 1 || !valid_m(ratio_m) || kv_dim < 1 || ik_dim < 0 || (tok_dtype != LCCA_F32 && tok_dtype != LCCA_BF16))
        return 0;
    const size_t esz = tok_dtype == LCCA_F32 ? 4 : 2;
    const size_t slots = (size_t)batch * ratio_m;
    const size_t logits = slots * sizeof(float);
    size_t n = up256(mul_sat(mul_sat(slots, (size_t)kv_dim), esz));                    // kv
    n = add_sat(n, up256(mul_sat(mul_sat(slots, (size_t)ik_dim), esz)));               // ik
    n = add_sat(n, ik_dim ? up256(logits) : logits);                                  // kv_logit
    if (ik_dim) n = add_sat(n, logits);                                               // ik_logit
    return n;
}

#ifdef LCCA_DEBUG
const char* lcca_version(void) { return "lcca 0.2.0 (gfx950, LCCA_DEBUG)"; }
#else
const char* lcca_version(void) { return "lcca 0.2.0 (gfx950)"; }
#endif

lcca_status lcca_debug_check(void* stream, uint32_t* bits) {
    g_err[0] = 0;
    if (bits) *bits = 0;
#ifdef LCCA_DEBUG
    uint32_t* w = nullptr;
    lcca_status s;
    if ((s = debug_word(&w))) return s;
    uint32_t v = 0;
    const hipStream_t st = (hipStream_t)stream;
    if ((s = hip_status(hipMemcpyAsync(&v, w, sizeof v, hipMemcpyDeviceToHost, st), "debug word read"))) return s;
    if ((s = hip_status(hipMemsetAsync(w, 0, sizeof v, st), "debug word clear"))) return s;
    if ((s = hip_status(hipStreamSynchronize(st), "debug word wait"))) return s;
    if (bits) *bits = v;
    if (v)
        return fail(LCCA_ERR_DEVICE_INDEX, "device indices out of range (bits 0x%x:%s%s%s)", v,
                    (v & LCCA_DBG_BLOCK) ? " block-table entry outside the pool;" : "",
                    (v & LCCA_DBG_ROW) ? " row_seq / row_pos outside batch / max_pos;" : "",
                    (v & LCCA_DBG_CHUNK) ? " cu_new / start_pos outside their contract;" : "");
    return LCCA_OK;
#else
    (void)stream;
    return fail(LCCA_ERR_UNSUPPORTED, "lcca_debug_check: this library was built without LCCA_DEBUG");
#endif
}

lcca_status lcca_rope(void* stream, int32_t dtype, void* x, int64_t rows, int32_t heads, int32_t dim,
                      int32_t rope_off, int32_t rope_dim, const int32_t* pos, double theta, const float* inv_freq,
                      int32_t flags) {
    g_err[0] = 0;
    if (dtype != LCCA_F32 && dtype != LCCA_BF16) return fail(LCCA_ERR_UNSUPPORTED, "rope: dtype %d (F32 or BF16)", dtype);
    if (rows < 0 || heads < 1 || dim < 1)
        return fail(LCCA_ERR_INVALID_ARG, "rope: rows=%lld heads=%d dim=%d", (long long)rows, heads, dim);
    if (rope_dim < 2 || rope_dim % 2 || rope_dim > lcca::kRopeMaxDim || rope_off < 0 ||
        (int64_t)rope_off + rope_dim > dim)
        return fail(LCCA_ERR_INVALID_ARG, "rope: slice [%d, %d + %d) of dim %d (even width 2..%d inside the vector)",
                    rope_off, rope_off, rope_dim, dim, lcca::kRopeMaxDim);
    if (flags & ~(LCCA_ROPE_HALF | LCCA_ROPE_INVERSE)) return fail(LCCA_ERR_INVALID_ARG, "rope: flags 0x%x", flags);
    if (!inv_freq && !(std::isfinite(theta) && theta > 0.0))
        return fail(LCCA_ERR_INVALID_ARG, "rope: theta=%g (finite and > 0 without inv_freq)", theta);
    if (mul_sat(mul_sat((size_t)rows, (size_t)heads), (size_t)dim) >= ((size_t)1 << 62))
        return fail(LCCA_ERR_INVALID_ARG, "rope: rows x heads x dim too large");
    if (rows == 0) return LCCA_OK;
    if (!x || !pos) return fail(LCCA_ERR_INVALID_ARG, "rope: x=%p pos=%p", x, (const void*)pos);
    lcca::RopeArgs a{};
    a.x = x; a.rows = rows; a.heads = heads; a.dim = dim; a.off = rope_off; a.rd = rope_dim; a.pos = pos;
    a.bf16 = dtype == LCCA_BF16;
    a.half_split = (flags & LCCA_ROPE_HALF) != 0;
    a.inverse = (flags & LCCA_ROPE_INVERSE) != 0;
    for (int i = 0; i < rope_dim / 2; ++i) {
        a.freq[i] = inv_freq ? inv_freq[i] : (float)std::pow(theta, -2.0 * i / rope_dim);
        if (!std::isfinite(a.freq[i])) return fail(LCCA_ERR_INVALID_ARG, "rope: frequency %d not finite", i);
    }
    return hip_status(lcca::launch_rope(a, (hipStream_t)stream), "rope launch");
}

const char* lcca_status_string(lcca_status s) {
    switch (s) {
    case LCCA_OK: return "ok";
    case LCCA_ERR_INVALID_ARG: return "invalid argument";
    case LCCA_ERR_UNSUPPORTED: return "unsupported dtype/shape combination";
    case LCCA_ERR_WORKSPACE: return "workspace missing or too small";
    case LCCA_ERR_HIP: return "HIP runtime error";
    case LCCA_ERR_DEVICE_INDEX: return "device-side index out of range (debug build)";
    }
    return "unknown status";
}

}  // extern "C"

namespace {

// Validation and kernel arguments of each stage, shared by its own entry
// point and by lcca_decode_select.
lcca_status prep_compress(const lcca_pages* pages, const int32_t* cu_new, const int32_t* start_pos, int32_t total_new,
                          int32_t tok_dtype, const void* kv_tok, const float* kv_logit, const void* ik_tok,
                          const float* ik_logit, const lcca_paged_cache* kv, const lcca_paged_cache* ik,
                          const lcca_window_cache* win, const lcca_remainder* rem, lcca::CompressArgs& a) {
    lcca_status s;
    if ((s = check_pages(pages))) return s;
    if ((s = check_pool(kv, "kv"))) return s;
    if (ik && (s = check_pool(ik, "ik"))) return s;
    if (win && (s = check_window(win, kv->dim))) return s;
    if (total_new < 0) return fail(LCCA_ERR_INVALID_ARG, "total_new=%d", total_new);
    if (!cu_new || !start_pos) return fail(LCCA_ERR_INVALID_ARG, "cu_new/start_pos NULL");
    if (tok_dtype != LCCA_F32 && tok_dtype != LCCA_BF16)
        return fail(LCCA_ERR_UNSUPPORTED, "token dtype %d (F32 or BF16)", tok_dtype);
    if (total_new > 0 && (!kv_tok || !kv_logit)) return fail(LCCA_ERR_INVALID_ARG, "kv_tok/kv_logit NULL");
    if (ik && total_new > 0 && (!ik_tok || !ik_logit)) return fail(LCCA_ERR_INVALID_ARG, "ik_tok/ik_logit NULL");
    if (!ik && (ik_tok || ik_logit)) return fail(LCCA_ERR_INVALID_ARG, "ik_tok given without an ik pool");
    if (kv->dtype == LCCA_FP8_E4M3) return fail(LCCA_ERR_UNSUPPORTED, "kv pool dtype FP8 (F32, BF16 or MXFP4)");
    if (ik && ik->dtype == LCCA_MXFP4) return fail(LCCA_ERR_UNSUPPORTED, "ik pool dtype MXFP4 (F32, BF16 or FP8)");
    if (ik && ik->dtype == LCCA_FP8_E4M3 && ik->scale)
        return fail(LCCA_ERR_UNSUPPORTED, "FP8 ik pool with a scale array (raw E4M3 only)");
    if (ik && ik->ratio_m != kv->ratio_m) return fail(LCCA_ERR_INVALID_ARG, "kv and ik ratio_m differ");
    if (kv->dim % 8 || (ik && ik->dim % 8)) return fail(LCCA_ERR_UNSUPPORTED, "dims must be multiples of 8");
    if (kv->dim > 2048) return fail(LCCA_ERR_UNSUPPORTED, "kv dim %d > 2048", kv->dim);
    if (!rem || rem->tok_dtype != tok_dtype || !rem->kv || !rem->kv_logit || (ik && (!rem->ik || !rem->ik_logit)))
        return fail(LCCA_ERR_INVALID_ARG, "remainder ring missing or of another token dtype");
    a = lcca::CompressArgs{};
    if ((s = debug_word(&a.dbg))) return s;
    a.block_table = pages->block_table; a.max_blocks = pages->max_blocks_per_seq;
    a.cu_new = cu_new; a.start_pos = start_pos; a.batch = pages->batch;
    a.total_new = total_new;
    a.n_blocks = ik ? std::min(kv->num_blocks, ik->num_blocks) : kv->num_blocks;
    a.tok_dtype = tok_dtype;
    a.kv_tok = kv_tok; a.kv_logit = kv_logit; a.ik_tok = ik ? ik_tok : nullptr; a.ik_logit = ik ? ik_logit : nullptr;
    a.m = kv->ratio_m; a.D = kv->dim; a.dI = ik ? ik->dim : 0;
    a.kv_dtype = kv->dtype; a.kv_data = kv->data; a.kv_scale = kv->scale;
    a.ik_dtype = ik ? ik->dtype : lcca::DT_NONE; a.ik_data = ik ? ik->data : nullptr; a.ik_scale = ik ? ik->scale : nullptr;
    a.win_dtype = win ? win->dtype : lcca::DT_NONE; a.win_cap = win ? win->capacity : 1;
    a.win_data = win ? win->data : nullptr; a.win_scale = win ? win->scale : nullptr;
    a.rem_kv = rem->kv; a.rem_ik = rem->ik; a.rem_kv_logit = rem->kv_logit; a.rem_ik_logit = rem->ik_logit;
    return LCCA_OK;
}

// `empty`: nothing to launch (no rows)
lcca_status prep_index(const lcca_pages* pages, const lcca_rows* rows, int32_t q_dtype, const void* q_idx,
                       int32_t HI, const float* w_idx, float s_I, const lcca_paged_cache* ik, float* logits,
                       int64_t ld, lcca::IndexArgs& a, int& max_entries, bool& empty) {
    lcca_status s;
    empty = false;
    if ((s = check_pages(pages))) return s;
    if ((s = check_pool(ik, "ik"))) return s;
    if ((s = check_rows(rows, ik->ratio_m, pages->max_blocks_per_seq))) return s;
    if (rows->num_rows == 0) { empty = true; return LCCA_OK; }
    if (!q_idx || !w_idx || !logits) return fail(LCCA_ERR_INVALID_ARG, "q_idx/w_idx/logits NULL");
    if (HI < 1) return fail(LCCA_ERR_INVALID_ARG, "HI=%d", HI);
    if (ik->dtype == LCCA_FP8_E4M3 && ik->scale)
        return fail(LCCA_ERR_UNSUPPORTED, "FP8 indexer keys with a scale array (raw E4M3 only)");
    const bool q8 = (q_dtype & LCCA_Q_FP8) != 0;
    q_dtype &= ~LCCA_Q_FP8;
    if (q8 && (q_dtype != LCCA_BF16 || ik->dtype != LCCA_FP8_E4M3 || rows->num_rows >= 64))
        return fail(LCCA_ERR_UNSUPPORTED, "FP8 queries (LCCA_Q_FP8): bf16 queries over FP8 keys, fewer than 64 rows");
    if (!lcca::index_supported(q_dtype, ik->dtype, HI, ik->dim))
        return fail(LCCA_ERR_UNSUPPORTED, "index_logits: q dtype %d, key dtype %d, HI=%d, dim=%d not built", q_dtype,
                    ik->dtype, HI, ik->dim);
    if (max_visible(rows->max_pos, ik->ratio_m) > INT32_MAX)
        return fail(LCCA_ERR_UNSUPPORTED, "index_logits: %lld visible entries", (long long)max_visible(rows->max_pos, 1));
    max_entries = (int)max_visible(rows->max_pos, ik->ratio_m);
    if (ld < max_entries) return fail(LCCA_ERR_INVALID_ARG, "ld=%lld < max visible entries %d", (long long)ld, max_entries);
    a = lcca::IndexArgs{};
    if ((s = debug_word(&a.dbg))) return s;
    a.block_table = pages->block_table; a.max_blocks = pages->max_blocks_per_seq;
    a.row_seq = rows->row_seq; a.row_pos = rows->row_pos; a.num_rows = rows->num_rows;
    a.batch = pages->batch; a.max_pos = rows->max_pos; a.n_blocks = ik->num_blocks;
    a.q = q_idx; a.w = w_idx; a.s_I = s_I; a.HI = HI; a.dI = ik->dim; a.m = ik->ratio_m; a.q8 = q8;
    a.key_dtype = ik->dtype; a.keys = ik->data; a.logits = logits; a.ld = ld;
    return LCCA_OK;
}

}  // namespace

extern "C" {

lcca_status lcca_compress_append(void* stream, const lcca_pages* pages, const int32_t* cu_new,
                                 const int32_t* start_pos, int32_t total_new, int32_t tok_dtype, const void* kv_tok,
                                 const float* kv_logit, const void* ik_tok, const float* ik_logit,
                                 const lcca_paged_cache* kv, const lcca_paged_cache* ik,
                                 const lcca_window_cache* win, const lcca_remainder* rem) {
    g_err[0] = 0;
    lcca::CompressArgs a;
    const lcca_status s = prep_compress(pages, cu_new, start_pos, total_new, tok_dtype, kv_tok, kv_logit, ik_tok,
                                        ik_logit, kv, ik, win, rem, a);
    if (s) return s;
    return hip_status(lcca::launch_compress_append(a, total_new, (hipStream_t)stream), "compress_append launch");
}

lcca_status lcca_compress_append_gated(void* stream, const lcca_pages* pages, const int32_t* cu_new,
                                       const int32_t* start_pos, int32_t total_new, int32_t tok_dtype,
                                       const void* kv_tok, const float* kv_logit, const void* ik_tok,
                                       const float* ik_logit, const lcca_paged_cache* kv, const lcca_paged_cache* ik,
                                       const lcca_window_cache* win, const lcca_remainder* rem) {
    g_err[0] = 0;
    lcca::CompressArgs a;
    const lcca_status s = prep_compress(pages, cu_new, start_pos, total_new, tok_dtype, kv_tok, kv_logit, ik_tok,
                                        ik_logit, kv, ik, win, rem, a);
    if (s) return s;
    a.gated = 1;
    return hip_status(lcca::launch_compress_gated(a, total_new, (hipStream_t)stream), "compress_append_gated launch");
}

lcca_status lcca_index_logits(void* stream, const lcca_pages* pages, const lcca_rows* rows, int32_t q_dtype,
                              const void* q_idx, int32_t HI, const float* w_idx, float s_I,
                              const lcca_paged_cache* ik, float* logits, int64_t ld) {
    g_err[0] = 0;
    lcca::IndexArgs a;
    int max_entries = 0;
    bool empty = false;
    const lcca_status s = prep_index(pages, rows, q_dtype, q_idx, HI, w_idx, s_I, ik, logits, ld, a, max_entries, empty);
    if (s || empty) return s;
    return hip_status(lcca::launch_index_logits(a, max_entries, (hipStream_t)stream), "index_logits launch");
}

size_t lcca_topk_workspace_size(const lcca_rows* rows, int32_t ratio_m, int32_t k) {
    if (!rows || rows->num_rows <= 0 || !valid_m(ratio_m) || k < 1 || rows->max_pos < 0) return 0;
    const int64_t nvis = max_visible(rows->max_pos, ratio_m);
    if (nvis > lcca::kTopkMaxEntries) return 0;                 // the selection itself is unsupported
    const int max_entries = (int)nvis;
    if (lcca::topk_slices(max_entries) == 1) return 0;
    return mul_sat(mul_sat((size_t)rows->num_rows, (size_t)lcca::topk_cand_stride(max_entries, k)), 8);
}

}  // extern "C"

namespace {

lcca_status prep_topk(const lcca_rows* rows, int32_t ratio_m, const float* logits, int64_t ld, int32_t k,
                      int32_t* topk_idx, void* ws, size_t ws_bytes, lcca::TopkArgs& a, int& max_entries, bool& empty) {
    lcca_status s;
    empty = false;
    if (!valid_m(ratio_m)) return fail(LCCA_ERR_INVALID_ARG, "ratio_m=%d", ratio_m);
    if ((s = check_rows(rows, ratio_m, 0))) return s;
    if (k < 1) return fail(LCCA_ERR_INVALID_ARG, "k=%d", k);
    if (rows->num_rows == 0) { empty = true; return LCCA_OK; }
    if (!logits || !topk_idx) return fail(LCCA_ERR_INVALID_ARG, "logits/topk_idx NULL");
    if (max_visible(rows->max_pos, ratio_m) > lcca::kTopkMaxEntries)
        return fail(LCCA_ERR_UNSUPPORTED, "%lld visible entries > %d", (long long)max_visible(rows->max_pos, ratio_m),
                    lcca::kTopkMaxEntries);
    max_entries = (int)max_visible(rows->max_pos, ratio_m);
    if (ld < max_entries) return fail(LCCA_ERR_INVALID_ARG, "ld=%lld < max visible entries %d", (long long)ld, max_entries);
    // the candidates' selection of long rows keeps a bitmap of its slices x k
    // candidates in the same LDS space as a row's
    if (lcca::topk_slices(max_entries) > 1 &&
        (int64_t)lcca::topk_slices(max_entries) * k > (int64_t)lcca::kTopkMaxEntries)
        return fail(LCCA_ERR_UNSUPPORTED, "%d slices x k=%d candidates > %d", lcca::topk_slices(max_entries), k,
                    lcca::kTopkMaxEntries);
    a = lcca::TopkArgs{};
    if ((s = debug_word(&a.dbg))) return s;
    a.row_pos = rows->row_pos; a.num_rows = rows->num_rows; a.m = ratio_m; a.max_pos = rows->max_pos;
    a.logits = logits; a.ld = ld; a.k = k; a.idx = topk_idx;
    if (lcca::topk_slices(max_entries) > 1) {
        const size_t need = lcca_topk_workspace_size(rows, ratio_m, k);
        if (!ws || ws_bytes < need)
            return fail(LCCA_ERR_WORKSPACE, "top-k of %d entries needs %zu workspace bytes (%zu given)", max_entries,
                        need, ws ? ws_bytes : (size_t)0);
        if (reinterpret_cast<uintptr_t>(ws) & 15) return fail(LCCA_ERR_INVALID_ARG, "top-k workspace not 16-byte aligned");
        a.cand_stride = lcca::topk_cand_stride(max_entries, k);
        a.cand_key = reinterpret_cast<uint32_t*>(ws);
        a.cand_idx = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + need / 2);
    }
    return LCCA_OK;
}

}  // namespace

extern "C" {

lcca_status lcca_topk_select(void* stream, const lcca_rows* rows, int32_t ratio_m, const float* logits, int64_t ld,
                             int32_t k, int32_t* topk_idx, void* ws, size_t ws_bytes) {
    g_err[0] = 0;
    lcca::TopkArgs a;
    int max_entries = 0;
    bool empty = false;
    const lcca_status s = prep_topk(rows, ratio_m, logits, ld, k, topk_idx, ws, ws_bytes, a, max_entries, empty);
    if (s || empty) return s;
    return hip_status(lcca::launch_topk_select(a, max_entries, (hipStream_t)stream), "topk_select launch");
}

size_t lcca_decode_select_workspace_size(const lcca_rows* rows, int32_t ratio_m, int32_t k) {
    if (!rows || rows->num_rows <= 0 || !valid_m(ratio_m) || k < 1 || rows->max_pos < 0) return 0;
    const int64_t nvis = max_visible(rows->max_pos, ratio_m);
    if (nvis > lcca::kTopkMaxEntries) return 0;                 // the selection itself is unsupported
    // the rows' leading-digit counts, after the slices' candidates when rows
    // are selected in two launches
    const size_t counts = (size_t)rows->num_rows * ((size_t)1 << lcca::kTopkLeadBits) * sizeof(uint32_t);
    if (lcca::topk_slices((int)nvis) > 1) return add_sat(lcca_topk_workspace_size(rows, ratio_m, k), counts);
    return counts;
}

lcca_status lcca_decode_select(void* stream, const lcca_pages* pages, const lcca_rows* rows, const int32_t* cu_new,
                               const int32_t* start_pos, int32_t total_new, int32_t tok_dtype, const void* kv_tok,
                               const float* kv_logit, const void* ik_tok, const float* ik_logit,
                               const lcca_paged_cache* kv, const lcca_paged_cache* ik, const lcca_window_cache* win,
                               const lcca_remainder* rem, int32_t q_dtype, const void* q_idx, int32_t HI,
                               const float* w_idx, float s_I, float* logits, int64_t ld, int32_t k,
                               int32_t* topk_idx, void* ws, size_t ws_bytes) {
    g_err[0] = 0;
    lcca_status s;
    if (!ik) return fail(LCCA_ERR_INVALID_ARG, "decode_select needs the indexer pool");
    lcca::CompressArgs c;
    if ((s = prep_compress(pages, cu_new, start_pos, total_new, tok_dtype, kv_tok, kv_logit, ik_tok, ik_logit, kv, ik,
                           win, rem, c)))
        return s;
    lcca::IndexArgs ia;
    int idx_entries = 0;
    bool empty = false;
    if ((s = prep_index(pages, rows, q_dtype, q_idx, HI, w_idx, s_I, ik, logits, ld, ia, idx_entries, empty))) return s;
    if (rows->num_rows != total_new || total_new != pages->batch)
        return fail(LCCA_ERR_INVALID_ARG, "decode_select: rows=%d, new tokens=%d, batch=%d (one new token and one row "
                    "per sequence)", rows->num_rows, total_new, pages->batch);
    if (empty) return LCCA_OK;
    lcca::TopkArgs ta;
    int sel_entries = 0;
    if ((s = prep_topk(rows, ik->ratio_m, logits, ld, k, topk_idx, ws, ws_bytes, ta, sel_entries, empty))) return s;
    if ((q_dtype & ~LCCA_Q_FP8) != LCCA_BF16 || rows->num_rows >= 64 || ik->ratio_m > 4 ||
        !lcca::topk_compress_supported(ta, sel_entries, tok_dtype))
        return fail(LCCA_ERR_UNSUPPORTED, "decode_select: needs bf16 queries and tokens, fewer than 64 rows, ratio_m "
                    "<= 4, 16-byte aligned logit rows, and rows of at most 32,768 entries or slices whose k "
                    "candidates total at most 32,768");
    {
        // the indexer counts the logits' leading key digits into the
        // workspace; one-launch selections read and clear them, two-launch
        // selections read them in every slice and clear them in the
        // candidates' selection
        const size_t need = lcca_decode_select_workspace_size(rows, ik->ratio_m, k);
        if (!ws || ws_bytes < need)
            return fail(LCCA_ERR_WORKSPACE, "decode_select needs %zu workspace bytes (%zu given)", need,
                        ws ? ws_bytes : (size_t)0);
        if (reinterpret_cast<uintptr_t>(ws) & 15)
            return fail(LCCA_ERR_INVALID_ARG, "decode_select workspace not 16-byte aligned");
        const size_t cand = lcca::topk_slices(sel_entries) > 1 ? lcca_topk_workspace_size(rows, ik->ratio_m, k) : 0;
        ia.lead_hist = ta.lead_hist = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ws) + cand);
    }
    ia.fresh = 1;
    ia.cu_new = cu_new; ia.start_pos = start_pos; ia.tok_dtype = tok_dtype;
    ia.ik_tok = ik_tok; ia.ik_logit = ik_logit; ia.rem_ik = rem->ik; ia.rem_ik_logit = rem->ik_logit;
    if ((s = hip_status(lcca::launch_index_logits(ia, idx_entries, (hipStream_t)stream), "index_logits launch")))
        return s;
    return hip_status(lcca::launch_topk_compress(ta, sel_entries, c, total_new, (hipStream_t)stream),
                      "topk_select + compress_append launch");
}

size_t lcca_sparse_attn_workspace_size(const lcca_rows* rows, int32_t ratio_m, int32_t H, int32_t dim, int32_t d_v,
                                       int32_t k, int32_t topk_given, int32_t window) {
    (void)dim;
    if (!rows || !valid_m(ratio_m) || rows->num_rows <= 0) return 0;
    return attn_plan(rows->num_rows, rows->max_pos, ratio_m, H, d_v, k, topk_given != 0, window).ws_bytes;
}

}  // extern "C"

namespace {

// The attention call with its partial states in `ws` (the caller's
// workspace), or, with `scratch` set, in the library's per-device scratch
// array, whose maximum size is checked against the plan before it is looked
// up.
lcca_status attn_call(void* stream, const lcca_pages* pages, const lcca_rows* rows, int32_t q_dtype, const void* q,
                      int32_t H, int32_t d_v, float sm_scale, const lcca_paged_cache* kv, const int32_t* topk_idx,
                      int32_t k, const lcca_window_cache* win, int32_t out_dtype, void* out, float* lse, void* ws,
                      size_t ws_bytes, bool scratch) {
    g_err[0] = 0;
    lcca_status s;
    if ((s = check_pages(pages))) return s;
    if ((s = check_pool(kv, "kv"))) return s;
    if ((s = check_rows(rows, kv->ratio_m, pages->max_blocks_per_seq))) return s;
    if ((s = check_window(win, kv->dim))) return s;
    if (rows->num_rows == 0) return LCCA_OK;
    if (!q || !out) return fail(LCCA_ERR_INVALID_ARG, "q/out NULL");
    if (H < 1 || d_v < 1 || d_v > kv->dim) return fail(LCCA_ERR_INVALID_ARG, "H=%d d_v=%d dim=%d", H, d_v, kv->dim);
    if (topk_idx && k < 1) return fail(LCCA_ERR_INVALID_ARG, "k=%d with a top-k index array", k);
    if (!std::isfinite(sm_scale)) return fail(LCCA_ERR_INVALID_ARG, "sm_scale not finite");
    if (out_dtype != LCCA_F32 && out_dtype != LCCA_BF16) return fail(LCCA_ERR_UNSUPPORTED, "out dtype %d", out_dtype);
    if (kv->dtype == LCCA_FP8_E4M3) return fail(LCCA_ERR_UNSUPPORTED, "FP8 kv pool (BF16, MXFP4 or F32)");
    const bool q8 = (q_dtype & LCCA_Q_FP8) != 0;
    const bool p16 = (q_dtype & LCCA_P_BF16) != 0;
    q_dtype &= ~(LCCA_Q_FP8 | LCCA_P_BF16);
    if (q8 && (q_dtype != LCCA_BF16 || kv->dtype != LCCA_MXFP4))
        return fail(LCCA_ERR_UNSUPPORTED, "sparse_attn: FP8 queries need BF16 q and an MXFP4 kv pool (q %d, kv %d)",
                    q_dtype, kv->dtype);
    if (!lcca::attn_supported(q_dtype, kv->dtype, win->dtype, H, kv->dim, d_v))
        return fail(LCCA_ERR_UNSUPPORTED, "sparse_attn: q %d, kv %d, window %d, H=%d, dim=%d, d_v=%d not built", q_dtype,
                    kv->dtype, win->dtype, H, kv->dim, d_v);
    const int m = kv->ratio_m;
    const bool f32 = q_dtype == LCCA_F32;
    AttnPlan plan = attn_plan(rows->num_rows, rows->max_pos, m, H, d_v, k, topk_idx != nullptr, win->window);
    if (!f32 && plan.split_tiles > lcca::attn_max_split_tiles())
        return fail(LCCA_ERR_UNSUPPORTED, "sparse_attn: %d key tiles per split needed (> %d)", plan.split_tiles,
                    lcca::attn_max_split_tiles());
    if (f32) {
        const int64_t L = (topk_idx ? (int64_t)k : max_visible(rows->max_pos, m)) +
                          std::min<int64_t>(win->window, (int64_t)rows->max_pos + 1);
        if (L > lcca::attn_f32_max_keys())
            return fail(LCCA_ERR_UNSUPPORTED, "fp32 attention: %lld keys per row > %d", (long long)L,
                        lcca::attn_f32_max_keys());
        plan = AttnPlan{1, 1, 0};
    }
    if (scratch && plan.ws_bytes > 0) {
        if (plan.ws_bytes > lcca::attn_scratch_bytes())
            return fail(LCCA_ERR_UNSUPPORTED, "sparse_attn_fwd_noalloc: partial states of %zu bytes exceed the %zu-byte "
                        "scratch array", plan.ws_bytes, lcca::attn_scratch_bytes());
        if ((s = hip_status(lcca::attn_scratch(&ws), "scratch array lookup"))) return s;
        ws_bytes = lcca::attn_scratch_bytes();
    }
    if (plan.ws_bytes > 0 && (!ws || ws_bytes < plan.ws_bytes))
        return fail(LCCA_ERR_WORKSPACE, "workspace %zu bytes at %p, need %zu", ws_bytes, ws, plan.ws_bytes);
    if (plan.ws_bytes > 0 && (reinterpret_cast<uintptr_t>(ws) & 15))
        return fail(LCCA_ERR_INVALID_ARG, "attention workspace not 16-byte aligned");
    lcca::AttnArgs a{};
    if ((s = debug_word(&a.dbg))) return s;
    a.block_table = pages->block_table; a.max_blocks = pages->max_blocks_per_seq;
    a.row_seq = rows->row_seq; a.row_pos = rows->row_pos; a.num_rows = rows->num_rows;
    a.batch = pages->batch; a.max_pos = rows->max_pos; a.n_blocks = kv->num_blocks;
    a.q = q; a.H = H; a.D = kv->dim; a.d_v = d_v; a.scale_log2 = sm_scale * 1.4426950408889634f;
    a.m = m; a.kv_dtype = kv->dtype; a.kv_data = kv->data; a.kv_scale = kv->scale;
    a.topk = topk_idx; a.k = topk_idx ? k : 0;
    a.win_dtype = win->dtype; a.win_data = win->data; a.win_scale = win->scale; a.win_cap = win->capacity;
    a.window = win->window;
    a.out_dtype = out_dtype; a.out = out; a.lse = lse;
    a.nsplit = plan.nsplit; a.split_tiles = plan.split_tiles;
    a.q8 = q8 ? 1 : 0;
    a.p_lo = p16 ? 0 : 1;
    if (plan.nsplit > 1) {
        const size_t parts = (size_t)rows->num_rows * plan.nsplit * H * d_v;
        const size_t po = (parts * sizeof(float) + 255) & ~(size_t)255;
        char* base = reinterpret_cast<char*>(ws);
        a.part_ml = reinterpret_cast<float*>(base + po);
        if (out_dtype == LCCA_BF16) {
            // fp16 partials (2 bytes per value) and their scales (one float
            // per 4 values) fit in the fp32 partials' place (4 bytes per value)
            const size_t ph = (parts * sizeof(uint16_t) + 255) & ~(size_t)255;
            a.part_h = reinterpret_cast<uint16_t*>(base);
            a.part_sc = reinterpret_cast<float*>(base + ph);
        } else {
            a.part_o = reinterpret_cast<float*>(base);
        }
    }
    return hip_status(lcca::launch_sparse_attn(a, (hipStream_t)stream), "sparse_attn launch");
}

}  // namespace

extern "C" {

lcca_status lcca_sparse_attn_fwd(void* stream, const lcca_pages* pages, const lcca_rows* rows, int32_t q_dtype,
                                 const void* q, int32_t H, int32_t d_v, float sm_scale, const lcca_paged_cache* kv,
                                 const int32_t* topk_idx, int32_t k, const lcca_window_cache* win, int32_t out_dtype,
                                 void* out, float* lse, void* ws, size_t ws_bytes) {
    return attn_call(stream, pages, rows, q_dtype, q, H, d_v, sm_scale, kv, topk_idx, k, win, out_dtype, out, lse, ws,
                     ws_bytes, false);
}

lcca_status lcca_sparse_attn_fwd_noalloc(void* stream, const lcca_pages* pages, const lcca_rows* rows,
                                         int32_t q_dtype, const void* q, int32_t H, int32_t d_v, float sm_scale,
                                         const lcca_paged_cache* kv, const int32_t* topk_idx, int32_t k,
                                         const lcca_window_cache* win, int32_t out_dtype, void* out, float* lse) {
    return attn_call(stream, pages, rows, q_dtype, q, H, d_v, sm_scale, kv, topk_idx, k, win, out_dtype, out, lse,
                     nullptr, 0, true);
}

}  // extern "C"
