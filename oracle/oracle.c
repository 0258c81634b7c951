/*
 * CPU oracle for compressed-KV attention: compress+append, indexer logits,
 * top-k selection and sparse attention over a paged compressed cache plus a
 * sliding window.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is plain, slow C with fp64 arithmetic.
 * It shares no code, header, table or constant with the HIP library and is
 * only loaded by the tests, by the smoke check and by the CPU-baseline leg of
 * the benchmark.  The product path never calls it.
 *
 * Sources (the only description of the method available):
 *   [P1] page "vLLM uveo DeepSeek V4 s 8,7x manjim KV cacheom: milijun tokena
 *        konteksta na standardnom GPU hardveru" (24-ai.news, Croatian); the
 *        German page "vLLM integriert DeepSeek V4 mit 8,7x kleinerem
 *        KV-Cache" is a line-for-line translation of it.
 *   [P3] page "DeepSeek-V4.1-Flash ve vLLM: kde se vzala 5,3x vyssi
 *        propustnost" (aidevelopers.cz, Czech).
 * The pages give prose, no formulas.  Where they are silent the plainest
 * reading is taken and stated next to the code that depends on it.
 *
 * Storage formats (shared byte layout with the device library, written
 * independently here):
 *   dtype 0 f32    : 4 bytes per element
 *   dtype 1 bf16   : 2 bytes, upper half of an IEEE binary32
 *   dtype 2 fp8    : 1 byte, OCP E4M3 "fn" (bias 7, max 448, no inf;
 *                    S.1111.111 is NaN)
 *   dtype 3 mxfp4  : OCP MX: E2M1 elements, two per byte (element 2i in the
 *                    low nibble), one E8M0 scale byte per 32 elements kept
 *                    in a separate scale array
 * Paged pools hold [num_blocks][E][row] with E = 256/m entries per block
 * (a block covers 256 logical token positions [P1 "Sto je vLLM morao
 * rijesiti u integraciji?"]).  Entry g of sequence b lives in physical block
 * block_table[b][g / E], slot g % E.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ODT_F32 = 0, ODT_BF16 = 1, ODT_FP8 = 2, ODT_MXFP4 = 3 };

/* ------------------------------------------------------------------------ */
/* Number formats                                                           */
/* ------------------------------------------------------------------------ */

static float bits_to_float(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t float_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

double orc_bf16_decode(uint16_t h) { return (double)bits_to_float((uint32_t)h << 16); }

/* Round an fp32 value to the nearest bf16, ties to the even bf16 code.
 * The two bf16 neighbours of x are its truncation `lo` and the next code
 * away from zero `lo + 1`; the discarded 16 bits say which is nearer. */
uint16_t orc_bf16_encode(float x)
{
    uint32_t u = float_to_bits(x);
    if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040u);       /* quiet NaN */
    uint32_t lo = u >> 16, rest = u & 0xFFFFu;
    if (rest > 0x8000u) return (uint16_t)(lo + 1);
    if (rest < 0x8000u) return (uint16_t)lo;
    return (uint16_t)((lo & 1u) ? lo + 1 : lo);                  /* exact tie */
}

/* E4M3 (OCP "fn"): value = (-1)^s * 2^(e-7) * (1 + m/8) for e >= 1,
 * (-1)^s * 2^-6 * (m/8) for e = 0; e = 15, m = 7 is NaN. */
double orc_fp8_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Nearest E4M3 value to x, ties to the code with an even mantissa,
 * saturating to +-448.  Works on the exact fp32 input: the spacing of E4M3
 * values in the binade [2^e, 2^(e+1)) is 2^(e-3), and 2^-9 below 2^-6. */
uint8_t orc_fp8_encode(float xf)
{
    if (isnan(xf)) return 0x7F;
    double x = (double)xf;
    uint8_t sign = (x < 0 || (x == 0 && signbit(x))) ? 0x80 : 0x00;
    double a = fabs(x);
    if (a >= 448.0) return sign | 0x7E;                       /* saturate */
    int e;
    if (a < ldexp(1.0, -6)) e = -6;                           /* subnormal binade */
    else { int ex; frexp(a, &ex); e = ex - 1; }               /* a in [2^e, 2^(e+1)) */
    double quantum = ldexp(1.0, e - 3);
    double q = nearbyint(a / quantum);                        /* RNE (default mode) */
    double v = q * quantum;                                   /* exact */
    if (v >= 448.0) return sign | 0x7E;
    if (v == 0.0) return sign;
    if (v < ldexp(1.0, -6)) return sign | (uint8_t)(v / ldexp(1.0, -9));
    int ex; frexp(v, &ex); int ev = ex - 1;                   /* v may have moved up a binade */
    int mant = (int)((v / ldexp(1.0, ev) - 1.0) * 8.0);
    return sign | (uint8_t)(((ev + 7) << 3) | mant);
}

/* FP8 query rows with a power-of-two scale (the low-precision indexer's
 * quantisation of the query; the pages name FP8 indexer keys [P3 "Vykon
 * neprinesl jeden kernel"] and give no rule for a quantised query, so the
 * plainest one is taken, the MX block-scale rule with one block per row and
 * the exponent lowered by one so no element saturates):
 * X = floor(log2(max_i |x_i|)) - 7, so the largest magnitude divided by 2^X
 * lies in [128, 256), below E4M3's 448; code_i = RNE E4M3 of x_i / 2^X.
 * A row of zeros takes X = -127.  X is clamped to [-127, 127]. */
void orc_quantize_fp8_rows(const float* x, int64_t nrows, int dim, uint8_t* codes, int32_t* X)
{
    for (int64_t r = 0; r < nrows; ++r) {
        const float* xr = x + r * dim;
        double amax = 0.0;
        for (int i = 0; i < dim; ++i) if (fabs((double)xr[i]) > amax) amax = fabs((double)xr[i]);
        int e = -127;
        if (amax > 0.0) {
            int ex; frexp(amax, &ex);                 /* amax in [2^(ex-1), 2^ex) */
            e = (ex - 1) - 7;
            if (e < -127) e = -127;
            if (e > 127) e = 127;
        }
        X[r] = e;
        for (int i = 0; i < dim; ++i) codes[r * dim + i] = orc_fp8_encode((float)ldexp((double)xr[i], -e));
    }
}

/* E2M1 nibble: s e e m; values 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double orc_fp4_decode(uint8_t nib)
{
    int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* Nearest E2M1 value to v (already divided by its block scale, exactly),
 * ties to the even mantissa, saturating to +-6. */
uint8_t orc_fp4_encode(double v)
{
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    uint8_t sign = (v < 0 || (v == 0 && signbit(v))) ? 8 : 0;
    double a = fabs(v);
    if (!(a < 6.0)) return sign | 7;                          /* saturate (and NaN) */
    int best = 0;
    for (int c = 1; c < 8; ++c) {
        double dc = fabs(mag[c] - a), db = fabs(mag[best] - a);
        if (dc < db || (dc == db && (c & 1) == 0)) best = c;
    }
    return sign | (uint8_t)best;
}

/* OCP MX block scale: X = floor(log2(amax)) - 2 (2 = exponent of the largest
 * E2M1 value), clamped to the E8M0 range [-127, 127]; amax = 0 gives -127.
 * The stored byte is X + 127. */
int orc_mx_scale_exp(float amax)
{
    if (!(amax > 0.0f)) return -127;
    int ex; frexp((double)amax, &ex);
    int X = (ex - 1) - 2;
    if (X < -127) X = -127;
    if (X > 127) X = 127;
    return X;
}

static int64_t row_bytes(int dtype, int dim)
{
    switch (dtype) {
    case ODT_F32: return 4LL * dim;
    case ODT_BF16: return 2LL * dim;
    case ODT_FP8: return dim;
    case ODT_MXFP4: return dim / 2;
    }
    return -1;
}

/* Read stored row `row` of a pool/ring as exact doubles (dequantised). */
static void load_row(int dtype, const void* data, const void* scale, int64_t row, int dim, double* out)
{
    const uint8_t* base = (const uint8_t*)data + row * row_bytes(dtype, dim);
    switch (dtype) {
    case ODT_F32:
        for (int i = 0; i < dim; ++i) { float f; memcpy(&f, base + 4 * i, 4); out[i] = f; }
        break;
    case ODT_BF16:
        for (int i = 0; i < dim; ++i) { uint16_t h; memcpy(&h, base + 2 * i, 2); out[i] = orc_bf16_decode(h); }
        break;
    case ODT_FP8: {
        double s = scale ? (double)((const float*)scale)[row] : 1.0;
        for (int i = 0; i < dim; ++i) out[i] = orc_fp8_decode(base[i]) * s;
        break;
    }
    case ODT_MXFP4: {
        const uint8_t* sc = (const uint8_t*)scale + row * (dim / 32);
        for (int i = 0; i < dim; ++i) {
            uint8_t byte = base[i / 2];
            uint8_t nib = (i & 1) ? (byte >> 4) : (byte & 15);
            out[i] = ldexp(orc_fp4_decode(nib), (int)sc[i / 32] - 127);
        }
        break;
    }
    }
}

/* Encode the fp32 vector x into stored row `row`.
 *   f32/bf16: cast (bf16 rounds to nearest even).
 *   fp8 with a scale array: per-row scale s = amax/448 (fp32 division; 1 if
 *     amax = 0), code = RNE(x/s) with the quotient taken in fp32, saturating.
 *   fp8 without a scale array: code = RNE(x), saturating.
 *   mxfp4: per 32-element block, the OCP MX scale and RNE E2M1 elements. */
static void store_row(int dtype, void* data, void* scale, int64_t row, int dim, const float* x)
{
    uint8_t* base = (uint8_t*)data + row * row_bytes(dtype, dim);
    switch (dtype) {
    case ODT_F32:
        memcpy(base, x, 4 * (size_t)dim);
        break;
    case ODT_BF16:
        for (int i = 0; i < dim; ++i) { uint16_t h = orc_bf16_encode(x[i]); memcpy(base + 2 * i, &h, 2); }
        break;
    case ODT_FP8:
        if (scale) {
            float amax = 0.0f;
            for (int i = 0; i < dim; ++i) if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
            float s = (amax > 0.0f) ? amax / 448.0f : 1.0f;
            ((float*)scale)[row] = s;
            for (int i = 0; i < dim; ++i) { float q = x[i] / s; base[i] = orc_fp8_encode(q); }
        } else {
            for (int i = 0; i < dim; ++i) base[i] = orc_fp8_encode(x[i]);
        }
        break;
    case ODT_MXFP4: {
        uint8_t* sc = (uint8_t*)scale + row * (dim / 32);
        memset(base, 0, (size_t)dim / 2);
        for (int blk = 0; blk < dim / 32; ++blk) {
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) { float a = fabsf(x[blk * 32 + i]); if (a > amax) amax = a; }
            int X = orc_mx_scale_exp(amax);
            sc[blk] = (uint8_t)(X + 127);
            for (int i = 0; i < 32; ++i) {
                int j = blk * 32 + i;
                uint8_t nib = orc_fp4_encode(ldexp((double)x[j], -X));
                base[j / 2] |= (j & 1) ? (uint8_t)(nib << 4) : nib;
            }
        }
        break;
    }
    }
}

void orc_store_rows(int dtype, void* data, void* scale, int64_t first_row, int64_t nrows, int dim, const float* x)
{
    for (int64_t r = 0; r < nrows; ++r) store_row(dtype, data, scale, first_row + r, dim, x + r * dim);
}

void orc_load_rows(int dtype, const void* data, const void* scale, int64_t first_row, int64_t nrows, int dim, double* out)
{
    for (int64_t r = 0; r < nrows; ++r) load_row(dtype, data, scale, first_row + r, dim, out + r * dim);
}

/* Token inputs are f32 or bf16; both convert to double exactly. */
static double tok_elem(int tok_dtype, const void* p, int64_t i)
{
    if (tok_dtype == ODT_F32) { float f; memcpy(&f, (const uint8_t*)p + 4 * i, 4); return f; }
    uint16_t h; memcpy(&h, (const uint8_t*)p + 2 * i, 2); return orc_bf16_decode(h);
}

static void tok_copy(int tok_dtype, const void* src, int64_t src_row, void* dst, int64_t dst_row, int dim)
{
    int64_t rb = (tok_dtype == ODT_F32 ? 4 : 2) * (int64_t)dim;
    memcpy((uint8_t*)dst + dst_row * rb, (const uint8_t*)src + src_row * rb, (size_t)rb);
}

/* Pool row of entry g of sequence b. */
static int64_t pool_row(const int32_t* block_table, int max_blocks, int m, int b, int64_t g)
{
    int E = 256 / m;
    int64_t blk = block_table[(int64_t)b * max_blocks + g / E];
    return blk * E + g % E;
}

/* ------------------------------------------------------------------------ */
/* Stage 1+2: compress (softmax-weighted aggregation of m tokens) + append   */
/* ------------------------------------------------------------------------ */

/* Softmax-weighted sum of one group of m token vectors, one scalar logit per
 * token [P1 "Kako funkcionira optimizacija KV cachea?": tokens are folded
 * by weighted summation; the weights are a softmax over the group's
 * per-token logits].  w_i = exp(a_i - mu) / sum_j exp(a_j - mu) with mu the
 * group maximum; C = sum_i w_i x_i, accumulated in i order, in fp64. */
void orc_group_compress(int m, int dim, const double* x /*[m][dim]*/, const double* a /*[m]*/, double* C)
{
    double mu = a[0];
    for (int i = 1; i < m; ++i) if (a[i] > mu) mu = a[i];
    double* w = (double*)malloc(sizeof(double) * (size_t)m);
    double S = 0.0;
    for (int i = 0; i < m; ++i) { w[i] = exp(a[i] - mu); S += w[i]; }
    for (int i = 0; i < m; ++i) w[i] /= S;
    for (int d = 0; d < dim; ++d) {
        double acc = 0.0;
        for (int i = 0; i < m; ++i) acc += w[i] * x[(int64_t)i * dim + d];
        C[d] = acc;
    }
    free(w);
}

/* The per-channel-gated variant: every channel d of every token carries its
 * own logit a[i][d], and the softmax runs over the group's m tokens for each
 * channel separately: w_id = exp(a_id - mu_d) / sum_j exp(a_jd - mu_d) with
 * mu_d the channel's group maximum, C_d = sum_i w_id x_id, accumulated in i
 * order, in fp64.  [P1 "Kako funkcionira optimizacija KV cachea?": tokens
 * are folded by weighted summation; weights per channel instead of per token
 * are the variant read R-1 names, the pages give no formula for either.]
 * With the same logit in every channel it is orc_group_compress. */
void orc_group_compress_gated(int m, int dim, const double* x /*[m][dim]*/, const double* a /*[m][dim]*/, double* C)
{
    double* w = (double*)malloc(sizeof(double) * (size_t)m);
    for (int d = 0; d < dim; ++d) {
        double mu = a[d];
        for (int i = 1; i < m; ++i) if (a[(int64_t)i * dim + d] > mu) mu = a[(int64_t)i * dim + d];
        double S = 0.0;
        for (int i = 0; i < m; ++i) { w[i] = exp(a[(int64_t)i * dim + d] - mu); S += w[i]; }
        double acc = 0.0;
        for (int i = 0; i < m; ++i) acc += (w[i] / S) * x[(int64_t)i * dim + d];
        C[d] = acc;
    }
    free(w);
}

/* Append a chunk of new tokens per sequence.
 *
 * Sequence b receives n_b = cu_new[b+1] - cu_new[b] tokens at positions
 * start_pos[b] .. start_pos[b] + n_b - 1.  For both streams (shared-KV
 * vectors, dim D; indexer keys, dim dI) every group g of m tokens that the
 * chunk completes is compressed and written to entry g of the paged pool.
 * Tokens of the group that precede the chunk come from the remainder ring,
 * slot t % m (the compressor remainder is held like sliding-window state
 * [P1 "Sto je vLLM morao rijesiti u integraciji?"]).  Tokens of a group that
 * stays incomplete are stored into that ring and produce no entry yet.
 * Every new token is also written, encoded, into the window ring at slot
 * t % win_cap (only the last win_cap tokens of a long chunk survive, so only
 * they are written).  A window of full vectors for recent positions sits
 * beside the compressed entries [P1 "Kako funkcionira ..."; FP8 window of 128
 * positions: P3 "Proc je obnova sliding-window cache draha"]. */
static int compress_append_impl(
    int gated,
    int batch, int max_blocks, const int32_t* block_table,
    const int32_t* cu_new, const int32_t* start_pos,
    int tok_dtype, const void* kv_tok, const float* kv_logit,
    const void* ik_tok, const float* ik_logit,
    int m, int D, int dI,
    int kv_dtype, void* kv_data, void* kv_scale,
    int ik_dtype, void* ik_data, void* ik_scale,
    int win_dtype, int win_cap, void* win_data, float* win_scale,
    void* rem_kv, void* rem_ik, float* rem_kv_logit, float* rem_ik_logit)
{
    if (m < 1 || 256 % m) return -1;
    int streams = (ik_tok && ik_data && dI > 0) ? 2 : 1;
    for (int b = 0; b < batch; ++b) {
        int64_t c0 = cu_new[b];
        int64_t n = cu_new[b + 1] - c0;
        int64_t start = start_pos[b], end = start + n;
        if (n <= 0) continue;
        /* groups completed by this chunk: g with start < (g+1)m <= end */
        int64_t g_first = start / m, g_end = end / m;
        for (int st = 0; st < streams; ++st) {
            int dim = st ? dI : D;
            const void* tok = st ? ik_tok : kv_tok;
            const float* lg = st ? ik_logit : kv_logit;
            const void* rtok = st ? rem_ik : rem_kv;
            const float* rlg = st ? rem_ik_logit : rem_kv_logit;
            int pdt = st ? ik_dtype : kv_dtype;
            void* pdata = st ? ik_data : kv_data;
            void* pscale = st ? ik_scale : kv_scale;
            /* logits per token, or per token and channel (gated) */
            const int la = gated ? dim : 1;
            double* x = (double*)malloc(sizeof(double) * (size_t)m * dim);
            double* a = (double*)malloc(sizeof(double) * (size_t)m * la);
            double* C = (double*)malloc(sizeof(double) * (size_t)dim);
            float* Cf = (float*)malloc(sizeof(float) * (size_t)dim);
            for (int64_t g = g_first; g < g_end; ++g) {
                for (int i = 0; i < m; ++i) {
                    int64_t t = g * m + i;
                    if (t >= start) {
                        int64_t row = c0 + (t - start);
                        for (int d = 0; d < dim; ++d) x[(int64_t)i * dim + d] = tok_elem(tok_dtype, tok, row * dim + d);
                        for (int d = 0; d < la; ++d) a[(int64_t)i * la + d] = lg[row * la + d];
                    } else {
                        int64_t row = (int64_t)b * m + t % m;
                        for (int d = 0; d < dim; ++d) x[(int64_t)i * dim + d] = tok_elem(tok_dtype, rtok, row * dim + d);
                        for (int d = 0; d < la; ++d) a[(int64_t)i * la + d] = rlg[row * la + d];
                    }
                }
                if (gated) orc_group_compress_gated(m, dim, x, a, C);
                else orc_group_compress(m, dim, x, a, C);
                /* The encoding decision is taken on the fp32 value. */
                for (int d = 0; d < dim; ++d) Cf[d] = (float)C[d];
                store_row(pdt, pdata, pscale, pool_row(block_table, max_blocks, m, b, g), dim, Cf);
            }
            free(x); free(a); free(C); free(Cf);
        }
        /* window ring: the last win_cap new tokens */
        if (win_data) {
            float* xf = (float*)malloc(sizeof(float) * (size_t)D);
            int64_t t0 = end - win_cap > start ? end - win_cap : start;
            for (int64_t t = t0; t < end; ++t) {
                int64_t row = c0 + (t - start);
                for (int d = 0; d < D; ++d) xf[d] = (float)tok_elem(tok_dtype, kv_tok, row * D + d);
                store_row(win_dtype, win_data, win_scale, (int64_t)b * win_cap + t % win_cap, D, xf);
            }
            free(xf);
        }
        /* remainder ring: new tokens of the incomplete last group */
        int64_t tail0 = (end / m) * m;
        if (tail0 < start) tail0 = start;
        for (int64_t t = tail0; t < end; ++t) {
            int64_t row = c0 + (t - start);
            int64_t slot = (int64_t)b * m + t % m;
            const int lk = gated ? D : 1, li = gated ? dI : 1;
            tok_copy(tok_dtype, kv_tok, row, rem_kv, slot, D);
            for (int d = 0; d < lk; ++d) rem_kv_logit[slot * lk + d] = kv_logit[row * lk + d];
            if (streams == 2) {
                tok_copy(tok_dtype, ik_tok, row, rem_ik, slot, dI);
                for (int d = 0; d < li; ++d) rem_ik_logit[slot * li + d] = ik_logit[row * li + d];
            }
        }
    }
    return 0;
}

int orc_compress_append(
    int batch, int max_blocks, const int32_t* block_table,
    const int32_t* cu_new, const int32_t* start_pos,
    int tok_dtype, const void* kv_tok, const float* kv_logit,
    const void* ik_tok, const float* ik_logit,
    int m, int D, int dI,
    int kv_dtype, void* kv_data, void* kv_scale,
    int ik_dtype, void* ik_data, void* ik_scale,
    int win_dtype, int win_cap, void* win_data, float* win_scale,
    void* rem_kv, void* rem_ik, float* rem_kv_logit, float* rem_ik_logit)
{
    return compress_append_impl(0, batch, max_blocks, block_table, cu_new, start_pos, tok_dtype, kv_tok, kv_logit,
                                ik_tok, ik_logit, m, D, dI, kv_dtype, kv_data, kv_scale, ik_dtype, ik_data, ik_scale,
                                win_dtype, win_cap, win_data, win_scale, rem_kv, rem_ik, rem_kv_logit, rem_ik_logit);
}

/* orc_compress_append with per-channel-gated groups (orc_group_compress_gated):
 * the logits are [n_new][D] and [n_new][dI], the remainder ring's logits
 * [batch][m][D] and [batch][m][dI]; everything else is unchanged. */
int orc_compress_append_gated(
    int batch, int max_blocks, const int32_t* block_table,
    const int32_t* cu_new, const int32_t* start_pos,
    int tok_dtype, const void* kv_tok, const float* kv_logit,
    const void* ik_tok, const float* ik_logit,
    int m, int D, int dI,
    int kv_dtype, void* kv_data, void* kv_scale,
    int ik_dtype, void* ik_data, void* ik_scale,
    int win_dtype, int win_cap, void* win_data, float* win_scale,
    void* rem_kv, void* rem_ik, float* rem_kv_logit, float* rem_ik_logit)
{
    return compress_append_impl(1, batch, max_blocks, block_table, cu_new, start_pos, tok_dtype, kv_tok, kv_logit,
                                ik_tok, ik_logit, m, D, dI, kv_dtype, kv_data, kv_scale, ik_dtype, ik_data, ik_scale,
                                win_dtype, win_cap, win_data, win_scale, rem_kv, rem_ik, rem_kv_logit, rem_ik_logit);
}

/* ------------------------------------------------------------------------ */
/* Stage 3: indexer logits (sparse MQA logits)                              */
/* ------------------------------------------------------------------------ */

/* Entry g is visible to a query at position p once its last token
 * (g+1)m - 1 <= p, so a row sees n = floor((p+1)/m) entries (causal
 * reading; the pages say only that the indexer scores candidate positions
 * [P3 "Vykon neprinesl jeden kernel"]). */
static int64_t visible_entries(int64_t p, int m) { return (p + 1) / m; }

static void load_vec(int dtype, const void* base, int64_t off, int dim, double* out)
{
    for (int d = 0; d < dim; ++d) out[d] = tok_elem(dtype, base, off + d);
}

/* l[r][g] = s_I * sum_h w[r][h] * max(0, q_I[r][h] . K_I[g]) for g < n_r:
 * per-head dot products of the indexer query with the compressed indexer
 * key, ReLU, then the per-head weighted sum (single shared key head, many
 * query heads).  Computed in fp64 on the dequantised stored keys. */
int orc_index_logits(
    int num_rows, const int32_t* row_seq, const int32_t* row_pos,
    int m, int max_blocks, const int32_t* block_table,
    int q_dtype, const void* q_idx, int HI, int dI, const float* w_idx, double s_I,
    int ik_dtype, const void* ik_data, const void* ik_scale,
    double* logits, int64_t ld)
{
    if (m < 1 || 256 % m) return -1;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < num_rows; ++r) {
        int b = row_seq[r];
        int64_t n = visible_entries(row_pos[r], m);
        double* q = (double*)malloc(sizeof(double) * (size_t)HI * dI);
        double* k = (double*)malloc(sizeof(double) * (size_t)dI);
        load_vec(q_dtype, q_idx, (int64_t)r * HI * dI, HI * dI, q);
        for (int64_t g = 0; g < n; ++g) {
            load_row(ik_dtype, ik_data, ik_scale, pool_row(block_table, max_blocks, m, b, g), dI, k);
            double l = 0.0;
            for (int h = 0; h < HI; ++h) {
                double dot = 0.0;
                for (int d = 0; d < dI; ++d) dot += q[(int64_t)h * dI + d] * k[d];
                l += (double)w_idx[(int64_t)r * HI + h] * (dot > 0.0 ? dot : 0.0);
            }
            logits[(int64_t)r * ld + g] = s_I * l;
        }
        free(q); free(k);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Stage 4: top-k selection                                                 */
/* ------------------------------------------------------------------------ */

typedef struct { double v; int64_t g; } orc_kv;

/* Descending value, then ascending index (so -0.0 and +0.0 tie). */
static int cmp_desc(const void* pa, const void* pb)
{
    const orc_kv* a = (const orc_kv*)pa; const orc_kv* b = (const orc_kv*)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->g > b->g) - (a->g < b->g);
}

static int cmp_i32(const void* pa, const void* pb)
{
    int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a > b) - (a < b);
}

/* S_r = the min(k, n_r) entries with the largest logits; equal logits are
 * ranked by smaller entry index.  Emitted in ascending entry order, padded
 * with -1 up to k.  Attention is restricted to these entries [P1 "Kako
 * funkcionira ...": the third tier limits computation to the top-k
 * compressed tokens]. */
int orc_topk(int num_rows, const int32_t* row_pos, int m, const double* logits, int64_t ld, int k, int32_t* idx)
{
    if (m < 1 || 256 % m) return -1;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < num_rows; ++r) {
        int64_t n = visible_entries(row_pos[r], m);
        orc_kv* all = (orc_kv*)malloc(sizeof(orc_kv) * (size_t)(n > 0 ? n : 1));
        for (int64_t g = 0; g < n; ++g) { all[g].v = logits[(int64_t)r * ld + g]; all[g].g = g; }
        qsort(all, (size_t)n, sizeof(orc_kv), cmp_desc);
        int64_t take = n < k ? n : k;
        int32_t* out = idx + (int64_t)r * k;
        for (int64_t i = 0; i < take; ++i) out[i] = (int32_t)all[i].g;
        qsort(out, (size_t)take, sizeof(int32_t), cmp_i32);
        for (int64_t i = take; i < k; ++i) out[i] = -1;
        free(all);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Stages 5+6: sparse attention over selected entries + window             */
/* ------------------------------------------------------------------------ */

/* For row r at position p with query heads q[h] (dim D):
 *   keys  = dequantised entries listed in topk_idx (entries -1 skipped; NULL
 *           means every visible entry 0..n_r-1), followed by the window
 *           tokens max(0, p-window+1) .. p read from ring slot t % win_cap;
 *   s_j   = sm_scale * q[h] . k_j;
 *   o[h]  = sum_j softmax(s)_j * v_j with v_j = k_j[0 : d_v]  (one vector is
 *           both key and value: shared KV [P1 "Kako funkcionira ..."]);
 *   lse[h]= log sum_j exp(s_j).
 * Compressed entries and window tokens enter one joint softmax (the two
 * tiers are merged, not gated).  fp64 throughout. */
int orc_sparse_attn(
    int num_rows, const int32_t* row_seq, const int32_t* row_pos,
    int m, int max_blocks, const int32_t* block_table,
    int q_dtype, const void* q, int H, int D, int d_v, double sm_scale,
    int kv_dtype, const void* kv_data, const void* kv_scale,
    const int32_t* topk_idx, int k,
    int win_dtype, int win_cap, int window, const void* win_data, const float* win_scale,
    double* out, double* lse)
{
    if (m < 1 || 256 % m || d_v > D) return -1;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < num_rows; ++r) {
        int b = row_seq[r];
        int64_t p = row_pos[r];
        int64_t n = visible_entries(p, m);
        int64_t nsel = topk_idx ? k : n;
        int64_t t0 = p - window + 1 > 0 ? p - window + 1 : 0;
        int64_t nwin = win_data ? p - t0 + 1 : 0;
        int64_t cap = nsel + nwin;
        double* K = (double*)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1) * D);
        int64_t nk = 0;
        for (int64_t i = 0; i < nsel; ++i) {
            int64_t g = topk_idx ? topk_idx[(int64_t)r * k + i] : i;
            if (g < 0 || g >= n) continue;      /* padding, or an entry the row cannot see yet */
            load_row(kv_dtype, kv_data, kv_scale, pool_row(block_table, max_blocks, m, b, g), D, K + nk * D);
            ++nk;
        }
        for (int64_t t = t0; t < t0 + nwin; ++t) {
            load_row(win_dtype, win_data, win_scale, (int64_t)b * win_cap + t % win_cap, D, K + nk * D);
            ++nk;
        }
        double* qh = (double*)malloc(sizeof(double) * (size_t)D);
        double* s = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        for (int h = 0; h < H; ++h) {
            load_vec(q_dtype, q, ((int64_t)r * H + h) * D, D, qh);
            double M = -INFINITY;
            for (int64_t j = 0; j < nk; ++j) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d) dot += qh[d] * K[j * D + d];
                s[j] = sm_scale * dot;
                if (s[j] > M) M = s[j];
            }
            double den = 0.0;
            for (int64_t j = 0; j < nk; ++j) { s[j] = exp(s[j] - M); den += s[j]; }
            double* o = out + ((int64_t)r * H + h) * d_v;
            for (int d = 0; d < d_v; ++d) {
                double acc = 0.0;
                for (int64_t j = 0; j < nk; ++j) acc += s[j] * K[j * D + d];
                o[d] = nk ? acc / den : 0.0;
            }
            if (lse) lse[(int64_t)r * H + h] = nk ? M + log(den) : -INFINITY;
        }
        free(K); free(qh); free(s);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Rotary position embedding of a slice of dimensions                        */
/* ------------------------------------------------------------------------ */

/* Rotation of the pairs of dims [off, off + rd) of every x[r][h][0..dim) by
 * the row's position [P1 "Kako funkcionira optimizacija KV cachea?": the
 * shared KV vectors carry RoPE dimensions and the output is rotated back].
 * The pages fix no convention, so it is the caller's: pair i < rd/2 is
 * (2i, 2i+1) with pairing 0 (interleaved) or (i, i + rd/2) with pairing 1
 * (half split); its frequency is freq[i] if freq is given, else
 * fp32(theta^(-2i/rd)); its angle is the fp32 product fp32(pos) * freq_i
 * (the angle a float pipeline forms), and the rotation by that angle (by its
 * negative with `inverse`) is done in fp64. */
void orc_rope(double* x, int64_t rows, int heads, int dim, int off, int rd, const int32_t* pos, double theta,
              const float* freq, int pairing, int inverse)
{
    int half = rd / 2;
    for (int64_t r = 0; r < rows; ++r) {
        for (int h = 0; h < heads; ++h) {
            double* v = x + (r * heads + h) * (int64_t)dim + off;
            for (int i = 0; i < half; ++i) {
                float f = freq ? freq[i] : (float)pow(theta, -2.0 * i / rd);
                float ang = (float)pos[r] * f;
                double c = cos((double)ang), s = sin((double)ang);
                if (inverse) s = -s;
                int ia = pairing ? i : 2 * i, ib = pairing ? i + half : 2 * i + 1;
                double a = v[ia], b = v[ib];
                v[ia] = a * c - b * s;
                v[ib] = a * s + b * c;
            }
        }
    }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the parallel loops that follow (timing only). */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* Element-wise array helpers for the codec tests                           */
/* ------------------------------------------------------------------------ */

void orc_bf16_encode_array(const float* x, int64_t n, uint16_t* out) { for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_encode(x[i]); }
void orc_bf16_decode_array(const uint16_t* h, int64_t n, double* out) { for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_decode(h[i]); }
void orc_fp8_encode_array(const float* x, int64_t n, uint8_t* out) { for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_encode(x[i]); }
void orc_fp8_decode_array(const uint8_t* c, int64_t n, double* out) { for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_decode(c[i]); }
void orc_fp4_encode_array(const double* v, int64_t n, uint8_t* out) { for (int64_t i = 0; i < n; ++i) out[i] = orc_fp4_encode(v[i]); }
void orc_fp4_decode_array(const uint8_t* c, int64_t n, double* out) { for (int64_t i = 0; i < n; ++i) out[i] = orc_fp4_decode(c[i]); }
