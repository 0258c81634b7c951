/*
 * The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (test
 * infrastructure; built and run by tests/test_sanitizers.py).
 *
 * The oracle's source is compiled into this driver as one translation unit.
 * Every buffer is allocated at exactly the size the oracle's contract states,
 * so a read or write one element past a pool, ring, token array or output
 * is an ASan report; signed overflow, bad shifts and misaligned loads are
 * UBSan reports.  The driver walks every storage dtype of every stream
 * through two appended chunks (the second one reads the remainder ring the
 * first left), the indexer, the top-k and the attention (top-k and dense),
 * plus every codec over its whole code space.  Values are checked elsewhere;
 * here only that every output is written and finite.
 */
#include "../../oracle/oracle.c"

#include <stdio.h>

static int failures = 0;
#define CHECK(c)                                                                \
    do {                                                                        \
        if (!(c)) {                                                             \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);     \
            ++failures;                                                         \
        }                                                                       \
    } while (0)

/* a small deterministic generator (xorshift32) for values in [-2, 2) */
static uint32_t rng_state = 2463534242u;
static float frand(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 17;
    rng_state ^= rng_state << 5;
    return (float)((rng_state >> 8) * (4.0 / 16777216.0) - 2.0);
}

static void* xalloc(size_t n) { void* p = malloc(n ? n : 1); memset(p, 0, n ? n : 1); return p; }

static int64_t rbytes(int dtype, int dim)
{
    return dtype == ODT_F32 ? 4LL * dim : dtype == ODT_BF16 ? 2LL * dim : dtype == ODT_FP8 ? dim : dim / 2;
}

static void fill_tokens(int tok_dtype, void* p, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        float x = frand();
        if (tok_dtype == ODT_F32) ((float*)p)[i] = x;
        else ((uint16_t*)p)[i] = orc_bf16_encode(x);
    }
}

static void codecs(void)
{
    for (int c = 0; c < 256; ++c) {
        double v = orc_fp8_decode((uint8_t)c);
        if (!isnan(v)) CHECK(orc_fp8_encode((float)v) == (uint8_t)c || v == 0.0);
    }
    for (int c = 0; c < 16; ++c) CHECK(orc_fp4_encode(orc_fp4_decode((uint8_t)c)) == c || c == 8);
    for (uint32_t h = 0; h < 65536; h += 7) {
        double v = orc_bf16_decode((uint16_t)h);
        if (!isnan(v)) CHECK(orc_bf16_encode((float)v) == h);
    }
    const float amax[] = {0.0f, 1e-45f, 1e-38f, 0.75f, 6.0f, 448.0f, 3.0e38f};
    for (unsigned i = 0; i < sizeof amax / sizeof amax[0]; ++i) {
        int X = orc_mx_scale_exp(amax[i]);
        CHECK(X >= -127 && X <= 127);
    }
}

/* One configuration end to end. */
static void run(int tok_dtype, int kv_dtype, int ik_dtype, int win_dtype, int m)
{
    const int batch = 2, D = 64, dI = 32, HI = 4, H = 2, d_v = 48, k = 8, window = 8, win_cap = 24;
    const int prior[2] = {0, 0};
    const int n1[2] = {37, 9}, n2[2] = {11, 14};          /* two chunks per sequence */
    const int max_len = 37 + 11;
    const int max_blocks = (max_len + 255) / 256 + 1;
    const int E = 256 / m;
    const int num_blocks = batch * max_blocks;
    int32_t* bt = xalloc(sizeof(int32_t) * batch * max_blocks);
    for (int i = 0; i < batch * max_blocks; ++i) bt[i] = (i * 7 + 3) % num_blocks;   /* a permutation */

    const int64_t pool_rows = (int64_t)num_blocks * E;
    void* kv = xalloc(pool_rows * rbytes(kv_dtype, D));
    void* kv_scale = kv_dtype == ODT_MXFP4 ? xalloc(pool_rows * (D / 32)) : NULL;
    void* ik = xalloc(pool_rows * rbytes(ik_dtype, dI));
    void* win = xalloc((int64_t)batch * win_cap * rbytes(win_dtype, D));
    float* win_scale = win_dtype == ODT_FP8 ? xalloc(sizeof(float) * batch * win_cap) : NULL;
    const int esz = tok_dtype == ODT_F32 ? 4 : 2;
    void* rem_kv = xalloc((size_t)batch * m * D * esz);
    void* rem_ik = xalloc((size_t)batch * m * dI * esz);
    float* rem_kv_logit = xalloc(sizeof(float) * batch * m);
    float* rem_ik_logit = xalloc(sizeof(float) * batch * m);

    for (int chunk = 0; chunk < 2; ++chunk) {
        const int* n = chunk ? n2 : n1;
        int32_t cu[3] = {0, n[0], n[0] + n[1]};
        int32_t sp[2] = {prior[0] + (chunk ? n1[0] : 0), prior[1] + (chunk ? n1[1] : 0)};
        const int total = cu[2];
        void* kv_tok = xalloc((size_t)total * D * esz);
        void* ik_tok = xalloc((size_t)total * dI * esz);
        float* kl = xalloc(sizeof(float) * total);
        float* il = xalloc(sizeof(float) * total);
        fill_tokens(tok_dtype, kv_tok, (int64_t)total * D);
        fill_tokens(tok_dtype, ik_tok, (int64_t)total * dI);
        for (int i = 0; i < total; ++i) { kl[i] = frand(); il[i] = frand(); }
        int s = orc_compress_append(batch, max_blocks, bt, cu, sp, tok_dtype, kv_tok, kl, ik_tok, il, m, D, dI,
                                    kv_dtype, kv, kv_scale, ik_dtype, ik, NULL, win_dtype, win_cap, win, win_scale,
                                    rem_kv, rem_ik, rem_kv_logit, rem_ik_logit);
        CHECK(s == 0);
        free(kv_tok); free(ik_tok); free(kl); free(il);
    }

    /* rows: every position of the second chunk of each sequence */
    const int rows = n2[0] + n2[1];
    int32_t* row_seq = xalloc(sizeof(int32_t) * rows);
    int32_t* row_pos = xalloc(sizeof(int32_t) * rows);
    int r = 0;
    for (int b = 0; b < batch; ++b)
        for (int i = 0; i < n2[b]; ++i, ++r) { row_seq[r] = b; row_pos[r] = n1[b] + i; }
    const int64_t ld = max_len / m;
    void* q_idx = xalloc((size_t)rows * HI * dI * esz);
    float* w_idx = xalloc(sizeof(float) * rows * HI);
    fill_tokens(tok_dtype, q_idx, (int64_t)rows * HI * dI);
    for (int i = 0; i < rows * HI; ++i) w_idx[i] = frand() + 2.0f;
    double* logits = xalloc(sizeof(double) * rows * ld);
    CHECK(orc_index_logits(rows, row_seq, row_pos, m, max_blocks, bt, tok_dtype, q_idx, HI, dI, w_idx, 0.5,
                           ik_dtype, ik, NULL, logits, ld) == 0);
    for (int i = 0; i < rows; ++i)
        for (int64_t g = 0; g < (row_pos[i] + 1) / m; ++g) CHECK(isfinite(logits[i * ld + g]));
    int32_t* idx = xalloc(sizeof(int32_t) * rows * k);
    CHECK(orc_topk(rows, row_pos, m, logits, ld, k, idx) == 0);
    for (int i = 0; i < rows * k; ++i) CHECK(idx[i] >= -1 && idx[i] < ld);

    void* q = xalloc((size_t)rows * H * D * esz);
    fill_tokens(tok_dtype, q, (int64_t)rows * H * D);
    double* out = xalloc(sizeof(double) * rows * H * d_v);
    double* lse = xalloc(sizeof(double) * rows * H);
    for (int dense = 0; dense < 2; ++dense) {
        CHECK(orc_sparse_attn(rows, row_seq, row_pos, m, max_blocks, bt, tok_dtype, q, H, D, d_v, 0.125, kv_dtype, kv,
                              kv_scale, dense ? NULL : idx, dense ? 0 : k, win_dtype, win_cap, window, win, win_scale,
                              out, lse) == 0);
        for (int i = 0; i < rows * H * d_v; ++i) CHECK(isfinite(out[i]));
        for (int i = 0; i < rows * H; ++i) CHECK(isfinite(lse[i]));
    }
    free(bt); free(kv); free(kv_scale); free(ik); free(win); free(win_scale); free(rem_kv); free(rem_ik);
    free(rem_kv_logit); free(rem_ik_logit); free(row_seq); free(row_pos); free(q_idx); free(w_idx); free(logits);
    free(idx); free(q); free(out); free(lse);
}

int main(void)
{
    codecs();
    const int toks[] = {ODT_F32, ODT_BF16};
    const int kvs[] = {ODT_F32, ODT_BF16, ODT_MXFP4};
    const int iks[] = {ODT_F32, ODT_BF16, ODT_FP8};
    const int wins[] = {ODT_F32, ODT_BF16, ODT_FP8};
    const int ms[] = {1, 4, 16};
    int cases = 0;
    for (int a = 0; a < 2; ++a)
        for (int b = 0; b < 3; ++b)
            for (int c = 0; c < 3; ++c)
                for (int d = 0; d < 3; ++d)
                    for (int e = 0; e < 3; ++e) {
                        run(toks[a], kvs[b], iks[c], wins[d], ms[e]);
                        ++cases;
                    }
    printf("oracle sanitizer run: %d configurations, %d failed checks\n", cases, failures);
    return failures ? 1 : 0;
}
