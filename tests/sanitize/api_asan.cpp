// The host side of liblcca under AddressSanitizer and UndefinedBehaviorSanitizer
// (test infrastructure; built and run by tests/test_sanitizers.py).
//
// lcca_api.cpp and the host code of every .hip file are compiled host-only
// with the sanitizers and linked into this driver.  It calls every entry
// point of include/lcca.h with argument sets that the host validation must
// reject -- each one is expected to return a specific status before any
// launch -- and sweeps the size functions over their whole argument range,
// extremes included, so signed overflow in the planning arithmetic or a bad
// format in an error message is a sanitizer report.  Device pointers are
// stand-in addresses that are never dereferenced: no case reaches a launch.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "../../include/lcca.h"

static int failures = 0;
static int checks = 0;

static void expect(lcca_status got, lcca_status want, int line) {
    ++checks;
    if (got != want) {
        std::fprintf(stderr, "line %d: status %d, expected %d (%s)\n", line, got, want, lcca_last_error());
        ++failures;
    }
}
#define EXPECT(call, want) expect((call), (want), __LINE__)

static void* const P = reinterpret_cast<void*>(0x10000);     // stand-in device address, never read
static int32_t* const PI = reinterpret_cast<int32_t*>(0x10000);
static float* const PF = reinterpret_cast<float*>(0x10000);

static lcca_paged_cache pool(int dtype, int dim, int m = 4, int blocks = 4) {
    return lcca_paged_cache{dtype, dim, m, blocks, P, dtype == LCCA_MXFP4 ? P : nullptr};
}

static void compress_cases() {
    lcca_pages pages{1, 4, PI};
    lcca_paged_cache kv = pool(LCCA_BF16, 576), ik = pool(LCCA_BF16, 128);
    lcca_window_cache win{LCCA_BF16, 576, 128, 128, P, nullptr};
    lcca_remainder rem{LCCA_BF16, P, P, PF, PF};
    auto call = [&](const lcca_pages* pg, int total, int tok, const lcca_paged_cache* k, const lcca_paged_cache* i,
                    const lcca_window_cache* w, const lcca_remainder* r) {
        return lcca_compress_append(nullptr, pg, PI, PI, total, tok, P, PF, i ? P : nullptr, i ? PF : nullptr, k, i,
                                    w, r);
    };
    EXPECT(call(nullptr, 4, LCCA_BF16, &kv, &ik, &win, &rem), LCCA_ERR_INVALID_ARG);
    lcca_pages bad_pages{0, 4, PI};
    EXPECT(call(&bad_pages, 4, LCCA_BF16, &kv, &ik, &win, &rem), LCCA_ERR_INVALID_ARG);
    EXPECT(call(&pages, -1, LCCA_BF16, &kv, &ik, &win, &rem), LCCA_ERR_INVALID_ARG);
    EXPECT(call(&pages, 4, LCCA_FP8_E4M3, &kv, &ik, &win, &rem), LCCA_ERR_UNSUPPORTED);
    lcca_paged_cache mx_ik = pool(LCCA_MXFP4, 128);
    EXPECT(call(&pages, 4, LCCA_BF16, &kv, &mx_ik, &win, &rem), LCCA_ERR_UNSUPPORTED);
    lcca_paged_cache fp8_kv = pool(LCCA_FP8_E4M3, 576);
    EXPECT(call(&pages, 4, LCCA_BF16, &fp8_kv, &ik, &win, &rem), LCCA_ERR_UNSUPPORTED);
    lcca_paged_cache odd = pool(LCCA_BF16, 580);
    lcca_window_cache odd_win{LCCA_BF16, 580, 128, 128, P, nullptr};
    EXPECT(call(&pages, 4, LCCA_BF16, &odd, &ik, &odd_win, &rem), LCCA_ERR_UNSUPPORTED);
    lcca_paged_cache m3 = pool(LCCA_BF16, 576, 3);
    EXPECT(call(&pages, 4, LCCA_BF16, &m3, &ik, &win, &rem), LCCA_ERR_INVALID_ARG);
    lcca_paged_cache ik8 = pool(LCCA_BF16, 128, 8);
    EXPECT(call(&pages, 4, LCCA_BF16, &kv, &ik8, &win, &rem), LCCA_ERR_INVALID_ARG);
    lcca_remainder rem32{LCCA_F32, P, P, PF, PF};
    EXPECT(call(&pages, 4, LCCA_BF16, &kv, &ik, &win, &rem32), LCCA_ERR_INVALID_ARG);
    EXPECT(call(&pages, 4, LCCA_BF16, &kv, &ik, &win, nullptr), LCCA_ERR_INVALID_ARG);
    lcca_window_cache small{LCCA_BF16, 576, 64, 128, P, nullptr};           // capacity < window
    EXPECT(call(&pages, 4, LCCA_BF16, &kv, &ik, &small, &rem), LCCA_ERR_INVALID_ARG);
    lcca_window_cache fp8_noscale{LCCA_FP8_E4M3, 576, 128, 128, P, nullptr};
    EXPECT(call(&pages, 4, LCCA_BF16, &kv, &ik, &fp8_noscale, &rem), LCCA_ERR_INVALID_ARG);
    lcca_paged_cache mx_noscale{LCCA_MXFP4, 576, 4, 4, P, nullptr};
    EXPECT(call(&pages, 4, LCCA_BF16, &mx_noscale, &ik, &win, &rem), LCCA_ERR_INVALID_ARG);
    // nothing to append: validated, then nothing launched
    EXPECT(call(&pages, 0, LCCA_BF16, &kv, &ik, &win, &rem), LCCA_OK);
}

static void index_topk_cases() {
    lcca_pages pages{1, 4, PI};
    lcca_rows rows{1, 100, PI, PI};
    lcca_paged_cache ik = pool(LCCA_BF16, 128);
    EXPECT(lcca_index_logits(nullptr, nullptr, &rows, LCCA_BF16, P, 64, PF, 1.0f, &ik, PF, 64), LCCA_ERR_INVALID_ARG);
    EXPECT(lcca_index_logits(nullptr, &pages, &rows, LCCA_BF16, P, 64, PF, 1.0f, &ik, PF, 10), LCCA_ERR_INVALID_ARG);
    EXPECT(lcca_index_logits(nullptr, &pages, &rows, LCCA_BF16, P, 48, PF, 1.0f, &ik, PF, 64), LCCA_ERR_UNSUPPORTED);
    EXPECT(lcca_index_logits(nullptr, &pages, &rows, LCCA_BF16, P, 0, PF, 1.0f, &ik, PF, 64), LCCA_ERR_INVALID_ARG);
    lcca_rows far{1, 4 * 256, PI, PI};
    EXPECT(lcca_index_logits(nullptr, &pages, &far, LCCA_BF16, P, 64, PF, 1.0f, &ik, PF, 4096), LCCA_ERR_INVALID_ARG);
    lcca_rows maxpos{1, INT_MAX, PI, PI};
    EXPECT(lcca_index_logits(nullptr, &pages, &maxpos, LCCA_BF16, P, 64, PF, 1.0f, &ik, PF, 64), LCCA_ERR_INVALID_ARG);
    lcca_rows negrows{-1, 100, PI, PI};
    EXPECT(lcca_index_logits(nullptr, &pages, &negrows, LCCA_BF16, P, 64, PF, 1.0f, &ik, PF, 64), LCCA_ERR_INVALID_ARG);
    lcca_paged_cache fp8s{LCCA_FP8_E4M3, 128, 4, 4, P, P};
    EXPECT(lcca_index_logits(nullptr, &pages, &rows, LCCA_BF16, P, 64, PF, 1.0f, &fp8s, PF, 64), LCCA_ERR_UNSUPPORTED);
    lcca_rows none{0, 0, PI, PI};
    EXPECT(lcca_index_logits(nullptr, &pages, &none, LCCA_BF16, P, 64, PF, 1.0f, &ik, PF, 64), LCCA_OK);

    EXPECT(lcca_topk_select(nullptr, &rows, 4, PF, 64, 0, PI, nullptr, 0), LCCA_ERR_INVALID_ARG);
    EXPECT(lcca_topk_select(nullptr, &rows, 3, PF, 64, 8, PI, nullptr, 0), LCCA_ERR_INVALID_ARG);
    EXPECT(lcca_topk_select(nullptr, &rows, 4, nullptr, 64, 8, PI, nullptr, 0), LCCA_ERR_INVALID_ARG);
    lcca_rows huge{1, 4 * (1 << 18) + 3, PI, PI};
    EXPECT(lcca_topk_select(nullptr, &huge, 4, PF, (1 << 18) + 1, 64, PI, nullptr, 0), LCCA_ERR_UNSUPPORTED);
    EXPECT(lcca_topk_select(nullptr, &maxpos, 1, PF, INT64_MAX, 64, PI, nullptr, 0), LCCA_ERR_UNSUPPORTED);
    lcca_rows long_rows{3, 4 * 40000 - 1, PI, PI};
    EXPECT(lcca_topk_select(nullptr, &long_rows, 4, PF, 40000, 2048, PI, nullptr, 0), LCCA_ERR_WORKSPACE);
    lcca_rows ok{1, 4 * (1 << 18) - 1, PI, PI};
    size_t need = lcca_topk_workspace_size(&ok, 4, 16385);
    EXPECT(lcca_topk_select(nullptr, &ok, 4, PF, 1 << 18, 16385, PI, P, need), LCCA_ERR_UNSUPPORTED);
    need = lcca_topk_workspace_size(&ok, 4, 16384);
    EXPECT(lcca_topk_select(nullptr, &ok, 4, PF, 1 << 18, 16384, PI, reinterpret_cast<void*>(0x10008), need),
           LCCA_ERR_INVALID_ARG);
    EXPECT(lcca_topk_select(nullptr, &none, 4, PF, 64, 64, PI, nullptr, 0), LCCA_OK);
}

static void decode_select_cases() {
    lcca_pages pages{16, 256, PI};
    lcca_paged_cache kv = pool(LCCA_BF16, 576, 4, 4096), ik = pool(LCCA_BF16, 128, 4, 4096);
    lcca_window_cache win{LCCA_FP8_E4M3, 576, 128, 128, P, PF};
    lcca_remainder rem{LCCA_BF16, P, P, PF, PF};
    lcca_rows rows{16, 65535, PI, PI};
    auto call = [&](const lcca_rows* rw, int total, int tok, const lcca_paged_cache* i, const lcca_remainder* r,
                    int64_t ld, const lcca_pages* pg, void* ws, size_t ws_bytes) {
        return lcca_decode_select(nullptr, pg, rw, PI, PI, total, tok, P, PF, P, PF, &kv, i, &win, r, LCCA_BF16, P, 64,
                                  PF, 1.0f, PF, ld, 2048, PI, ws, ws_bytes);
    };
    EXPECT(call(&rows, 15, LCCA_BF16, &ik, &rem, 16384, &pages, nullptr, 0), LCCA_ERR_INVALID_ARG);
    EXPECT(call(&rows, 16, LCCA_BF16, nullptr, &rem, 16384, &pages, nullptr, 0), LCCA_ERR_INVALID_ARG);
    EXPECT(call(&rows, 16, LCCA_BF16, &ik, &rem, 16384, &pages, nullptr, 0), LCCA_ERR_WORKSPACE);
    const size_t need = lcca_decode_select_workspace_size(&rows, 4, 2048);
    EXPECT(call(&rows, 16, LCCA_BF16, &ik, &rem, 16384, &pages, reinterpret_cast<void*>(0x10008), need),
           LCCA_ERR_INVALID_ARG);
    lcca_remainder rem32{LCCA_F32, P, P, PF, PF};
    EXPECT(call(&rows, 16, LCCA_F32, &ik, &rem32, 16384, &pages, nullptr, 0), LCCA_ERR_UNSUPPORTED);
    EXPECT(call(&rows, 16, LCCA_BF16, &ik, &rem, 16386, &pages, nullptr, 0), LCCA_ERR_UNSUPPORTED);
}

static void attn_cases() {
    lcca_pages pg{16, 256, PI};
    lcca_rows rw{16, 65535, PI, PI};
    lcca_paged_cache kv = pool(LCCA_BF16, 576, 4, 4096);
    lcca_window_cache win{LCCA_FP8_E4M3, 576, 128, 128, P, PF};
    const size_t need = lcca_sparse_attn_workspace_size(&rw, 4, 64, 576, 576, 2048, 1, 128);
    EXPECT(need > 0 ? LCCA_OK : LCCA_ERR_INVALID_ARG, LCCA_OK);
    auto call = [&](const lcca_rows* r, int q_dt, int H, int d_v, float scale, const lcca_paged_cache* k,
                    const lcca_window_cache* w, int out_dt, void* ws, size_t ws_bytes) {
        return lcca_sparse_attn_fwd(nullptr, &pg, r, q_dt, P, H, d_v, scale, k, PI, 2048, w, out_dt, P, nullptr, ws,
                                    ws_bytes);
    };
    EXPECT(call(&rw, LCCA_BF16, 64, 576, 0.04f, &kv, &win, LCCA_F32, P, need - 1), LCCA_ERR_WORKSPACE);
    EXPECT(call(&rw, LCCA_BF16, 64, 576, 0.04f, &kv, &win, LCCA_F32, reinterpret_cast<void*>(0x10008), need),
           LCCA_ERR_INVALID_ARG);
    lcca_window_cache noscale{LCCA_FP8_E4M3, 576, 128, 128, P, nullptr};
    EXPECT(call(&rw, LCCA_BF16, 64, 576, 0.04f, &kv, &noscale, LCCA_F32, P, need), LCCA_ERR_INVALID_ARG);
    EXPECT(call(&rw, LCCA_BF16, 64, 577, 0.04f, &kv, &win, LCCA_F32, P, need), LCCA_ERR_INVALID_ARG);
    EXPECT(call(&rw, LCCA_BF16, 0, 576, 0.04f, &kv, &win, LCCA_F32, P, need), LCCA_ERR_INVALID_ARG);
    EXPECT(call(&rw, LCCA_BF16, 64, 576, __builtin_inff(), &kv, &win, LCCA_F32, P, need), LCCA_ERR_INVALID_ARG);
    EXPECT(call(&rw, LCCA_BF16, 64, 576, 0.04f, &kv, &win, LCCA_FP8_E4M3, P, need), LCCA_ERR_UNSUPPORTED);
    EXPECT(call(&rw, LCCA_BF16, 48, 576, 0.04f, &kv, &win, LCCA_F32, P, need), LCCA_ERR_UNSUPPORTED);
    lcca_paged_cache fp8 = pool(LCCA_FP8_E4M3, 576, 4, 4096);
    EXPECT(call(&rw, LCCA_BF16, 64, 576, 0.04f, &fp8, &win, LCCA_F32, P, need), LCCA_ERR_UNSUPPORTED);
    lcca_window_cache wrongdim{LCCA_FP8_E4M3, 512, 128, 128, P, PF};
    EXPECT(call(&rw, LCCA_BF16, 64, 576, 0.04f, &kv, &wrongdim, LCCA_F32, P, need), LCCA_ERR_INVALID_ARG);
    lcca_rows big{100, (1 << 20) - 1, PI, PI};
    lcca_pages bigpg{100, 4096, PI};
    lcca_paged_cache hca = pool(LCCA_BF16, 576, 128, 4096 * 100);
    EXPECT(lcca_sparse_attn_fwd_noalloc(nullptr, &bigpg, &big, LCCA_BF16, P, 640, 576, 0.04f, &hca, nullptr, 0, &win,
                                        LCCA_F32, P, nullptr),
           LCCA_ERR_UNSUPPORTED);
    lcca_rows none{0, 0, PI, PI};
    EXPECT(call(&none, LCCA_BF16, 64, 576, 0.04f, &kv, &win, LCCA_F32, nullptr, 0), LCCA_OK);
    // FP8 queries: an MXFP4 pool and bf16 queries only
    EXPECT(call(&rw, LCCA_BF16 | LCCA_Q_FP8, 64, 576, 0.04f, &kv, &win, LCCA_F32, P, need), LCCA_ERR_UNSUPPORTED);
    lcca_paged_cache mx = pool(LCCA_MXFP4, 576, 4, 4096);
    EXPECT(call(&rw, LCCA_F32 | LCCA_Q_FP8, 64, 576, 0.04f, &mx, &win, LCCA_F32, P, need), LCCA_ERR_UNSUPPORTED);
    // bf16-only weights: the flag does not lift the FP8-query rules, and other bits stay unsupported
    EXPECT(call(&rw, LCCA_BF16 | LCCA_Q_FP8 | LCCA_P_BF16, 64, 576, 0.04f, &kv, &win, LCCA_F32, P, need),
           LCCA_ERR_UNSUPPORTED);
    EXPECT(call(&rw, LCCA_BF16 | LCCA_P_BF16 | 0x400, 64, 576, 0.04f, &kv, &win, LCCA_F32, P, need),
           LCCA_ERR_UNSUPPORTED);
    EXPECT(call(&none, LCCA_BF16 | LCCA_P_BF16, 64, 576, 0.04f, &kv, &win, LCCA_F32, nullptr, 0), LCCA_OK);
}

static void rope_cases() {
    auto call = [](int dt, int64_t rows, int heads, int dim, int off, int rd, double theta, const float* fr,
                   int flags) { return lcca_rope(nullptr, dt, P, rows, heads, dim, off, rd, PI, theta, fr, flags); };
    EXPECT(call(LCCA_FP8_E4M3, 4, 2, 64, 0, 64, 1e4, nullptr, 0), LCCA_ERR_UNSUPPORTED);
    EXPECT(call(LCCA_F32, 4, 2, 64, 0, 63, 1e4, nullptr, 0), LCCA_ERR_INVALID_ARG);
    EXPECT(call(LCCA_F32, 4, 2, 64, INT_MAX, 64, 1e4, nullptr, 0), LCCA_ERR_INVALID_ARG);
    EXPECT(call(LCCA_F32, 4, 2, 600, 0, 258, 1e4, nullptr, 0), LCCA_ERR_INVALID_ARG);
    EXPECT(call(LCCA_F32, INT64_MAX, INT_MAX, INT_MAX, 0, 64, 1e4, nullptr, 0), LCCA_ERR_INVALID_ARG);
    EXPECT(call(LCCA_F32, -1, 2, 64, 0, 64, 1e4, nullptr, 0), LCCA_ERR_INVALID_ARG);
    EXPECT(call(LCCA_BF16, 4, 2, 64, 0, 64, 0.0, nullptr, 0), LCCA_ERR_INVALID_ARG);
    EXPECT(call(LCCA_BF16, 4, 2, 64, 0, 64, 1e4, nullptr, 8), LCCA_ERR_INVALID_ARG);
    const float inf_table[2] = {1.0f, __builtin_inff()};
    EXPECT(call(LCCA_F32, 4, 2, 64, 0, 4, 1e4, inf_table, 0), LCCA_ERR_INVALID_ARG);
    EXPECT(call(LCCA_F32, 0, 2, 64, 0, 64, 1e4, nullptr, LCCA_ROPE_HALF | LCCA_ROPE_INVERSE), LCCA_OK);
}

// Size functions over their argument range: each returns a size (0 for an
// invalid argument) without overflowing.
static void size_sweeps() {
    const int32_t counts[] = {INT_MIN, -1, 0, 1, 7, 64, 65535, 1 << 20, INT_MAX - 1, INT_MAX};
    const int32_t ms[] = {-4, 0, 1, 3, 4, 128, 256, 512};
    for (int32_t n : counts)
        for (int32_t mp : counts)
            for (int32_t m : ms) {
                lcca_rows rw{n, mp, PI, PI};
                for (int32_t k : counts) {
                    (void)lcca_topk_workspace_size(&rw, m, k);
                    (void)lcca_decode_select_workspace_size(&rw, m, k);
                }
                for (int32_t h : {1, 64, 640, INT_MAX})
                    for (int32_t dv : {1, 512, 576, INT_MAX})
                        for (int32_t k : {0, 64, 2048, INT_MAX})
                            for (int32_t w : {0, 128, INT_MAX}) {
                                (void)lcca_sparse_attn_workspace_size(&rw, m, h, 576, dv, k, 1, w);
                                (void)lcca_sparse_attn_workspace_size(&rw, m, h, 576, dv, k, 0, w);
                            }
            }
    (void)lcca_topk_workspace_size(nullptr, 4, 64);
    (void)lcca_sparse_attn_workspace_size(nullptr, 4, 64, 576, 576, 64, 1, 128);
    for (int32_t b : counts)
        for (int32_t m : ms)
            for (int32_t d : counts)
                for (int32_t di : counts)
                    for (int32_t t : {-1, 0, 1, 2, 3, 4}) (void)lcca_remainder_bytes(b, m, d, di, t);
    ++checks;
}

int main() {
    compress_cases();
    index_topk_cases();
    decode_select_cases();
    attn_cases();
    rope_cases();
    size_sweeps();
    for (int s = -6; s <= 1; ++s) (void)std::strlen(lcca_status_string(s));
    uint32_t bits = 5;
    EXPECT(lcca_debug_check(nullptr, &bits), LCCA_ERR_UNSUPPORTED);
    EXPECT(bits == 0 ? LCCA_OK : LCCA_ERR_INVALID_ARG, LCCA_OK);
    std::printf("api sanitizer run (%s): %d checks, %d failed\n", lcca_version(), checks, failures);
    return failures ? 1 : 0;
}
