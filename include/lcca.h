/*
 * lcca.h -- compressed-KV attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of liblcca.so: the four stages of decode and chunked-prefill
 * attention over a compressed, paged KV cache plus a sliding window.
 *
 * Sources for what each call computes:
 *   [P1] page "vLLM uveo DeepSeek V4 s 8,7x manjim KV cacheom: milijun
 *        tokena konteksta na standardnom GPU hardveru" (24-ai.news; the
 *        German page "vLLM integriert DeepSeek V4 mit 8,7x kleinerem
 *        KV-Cache" is its translation).
 *   [P3] page "DeepSeek-V4.1-Flash ve vLLM: kde se vzala 5,3x vyssi
 *        propustnost" (aidevelopers.cz).
 *
 * Conventions common to every call
 *   - Every buffer pointer is a DEVICE pointer owned by the caller, except
 *     the descriptor structs themselves, which live in host memory and are
 *     read during the call only.  The library never allocates, frees or
 *     synchronises.  Every call is asynchronous on `stream` (a hipStream_t;
 *     NULL is the null stream).
 *   - The library keeps no state between calls: positions and lengths are
 *     explicit, so a call repeated at the same positions rewrites the same
 *     bytes.
 *   - Arguments are validated on the host before any launch; a failing call
 *     launches nothing and returns a negative lcca_status, with details in
 *     lcca_last_error() (thread-local).  Indices that live in device memory
 *     (block-table entries, row_seq, row_pos, cu_new, start_pos) cannot be
 *     seen by the host: the release library uses them as given, and values
 *     outside their contract make kernels read or write outside the
 *     buffers.  The debug library (liblcca_debug.so, built with LCCA_DEBUG)
 *     checks each of them on the device before it forms an address, uses a
 *     value inside the range instead of a bad one, and records the violation
 *     for lcca_debug_check() (see there).  Top-k indices need no such check:
 *     entries < 0 or >= the row's visible count are skipped by contract.
 *
 * Data layout
 *   dtype codes: LCCA_F32 (4 B), LCCA_BF16 (2 B), LCCA_FP8_E4M3 (1 B, OCP
 *   E4M3 "fn": bias 7, max 448, no infinities), LCCA_MXFP4 (OCP MX: E2M1
 *   codes, two per byte with element 2i in the low nibble, and one E8M0
 *   scale byte per 32 elements in a separate array).
 *
 *   Paged pool (lcca_paged_cache): a block covers 256 logical token
 *   positions, so it holds E = 256 / ratio_m compressed entries [P1 "Sto je
 *   vLLM morao rijesiti u integraciji?": fixed logical blocks of 256 token
 *   positions, with a logical->physical mapping that depends on the layer's
 *   compression ratio].  data is [num_blocks][E][row] with row = dim
 *   elements of `dtype`; scale is [num_blocks][E][dim/32] E8M0 bytes for
 *   MXFP4, or [num_blocks][E] float (per-entry scale; NULL means 1) for FP8.
 *   Entry g of sequence b is at physical block block_table[b][g / E], slot
 *   g % E.
 *
 *   Window ring (lcca_window_cache): data [batch][capacity][dim]; token at
 *   position t of sequence b lives in slot t % capacity.  A query row at
 *   position p reads slots of positions p - window + 1 .. p, so every row
 *   attended after a chunk of n new tokens was appended needs those
 *   positions still in the ring: capacity >= window + n - 1 when rows
 *   inside the chunk are attended (chunked prefill), capacity >= window when
 *   only the chunk's last position is (decode).  A smaller ring gives early
 *   rows of the chunk the later tokens that overwrote their slots, silently.
 *   FP8 windows carry a float scale per slot [batch][capacity]: code = RNE(x / s) with
 *   s = max|x| / 448 (1 if the token is zero).  A window of full vectors of
 *   the most recent positions sits beside the compressed entries [P1 "Kako
 *   funkcionira optimizacija KV cachea?"; FP8, 128 positions: P3 "Proc je
 *   obnova sliding-window cache draha"].
 *
 *   Remainder ring (lcca_remainder): tokens of a sequence's incomplete last
 *   group, in the token dtype, [batch][ratio_m][dim], slot t % ratio_m, with
 *   float logits [batch][ratio_m]; the compressor's remainder is carried as
 *   window-like state [P1 "Sto je vLLM morao rijesiti u integraciji?"].
 *
 *   Query rows (lcca_rows): one row is one (sequence, position) with all its
 *   query heads.  A row at position p sees compressed entries
 *   g < n = floor((p + 1) / ratio_m) (an entry is visible once its last
 *   token is) and window tokens max(0, p - window + 1) .. p.
 */
#ifndef LCCA_H
#define LCCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t lcca_status;
#define LCCA_OK               0
#define LCCA_ERR_INVALID_ARG (-1)   /* NULL/negative/inconsistent argument          */
#define LCCA_ERR_UNSUPPORTED (-2)   /* dtype or shape combination not built          */
#define LCCA_ERR_WORKSPACE   (-3)   /* workspace missing or smaller than required    */
#define LCCA_ERR_HIP         (-4)   /* a HIP runtime call or kernel launch failed    */
#define LCCA_ERR_DEVICE_INDEX (-5)  /* debug build: a device-side index was out of range */

/* Bits of the debug library's device error word (lcca_debug_check). */
#define LCCA_DBG_BLOCK 1u   /* a block-table entry read outside [0, pool num_blocks)     */
#define LCCA_DBG_ROW   2u   /* row_seq outside [0, batch) or row_pos outside [0, max_pos] */
#define LCCA_DBG_CHUNK 4u   /* cu_new / start_pos of compress_append outside their contract:
                               cu_new[b] <= t < cu_new[b+1] <= total_new fails for a new
                               token t, start_pos[b] < 0, or the chunk ends beyond the
                               block table (max_blocks_per_seq * 256 positions)          */

typedef enum { LCCA_F32 = 0, LCCA_BF16 = 1, LCCA_FP8_E4M3 = 2, LCCA_MXFP4 = 3 } lcca_dtype;

/* Flag OR-ed into the q_dtype of lcca_index_logits and lcca_decode_select
 * (with LCCA_BF16 queries over raw FP8 E4M3 keys, fewer than 64 rows) and of
 * lcca_sparse_attn_fwd(_noalloc) (LCCA_BF16 queries, MXFP4 kv pool): the
 * kernel quantises each row's query per head to FP8 E4M3 with a power-of-two
 * scale, X = floor(log2 max_d |q_hd|) - 7 (the head's largest magnitude /
 * 2^X lies in [128, 256), so nothing saturates; X = -127 for a zero head),
 * q8_hd = RNE E4M3 of q_hd / 2^X, and computes q8_h . K_g * 2^X exactly on
 * the FP8 matrix cores (fp32 accumulation).  The logits are then those of
 * the quantised query; against the bf16 query each head's dot product moves
 * by at most sum_d max(2^-4 |q_hd|, 2^(X-10)) |K_gd|.  In the attention the
 * pool entries are scored by the scaled FP4 x FP8 matrix instructions
 * straight from the pool's E2M1 codes and E8M0 block scales, window tokens
 * by bf16 products with the same dequantised query q8 * 2^X, so every key
 * of the one softmax sees the quantised query; values stay as before.
 * [P3 "Vykon neprinesl jeden kernel": FP8 indexer keys, and a fused
 * attention reading a 4-bit KV cache; the query's quantisation rule is this
 * library's.] */
#define LCCA_Q_FP8 0x100

/* Flag OR-ed into the q_dtype of lcca_sparse_attn_fwd(_noalloc) (BF16 and
 * FP8-query paths; no effect on the F32 path): the softmax weights P enter
 * the P.V products as bf16 alone instead of a bf16 hi + lo pair (16
 * significant bits), which halves the P.V matrix work.  Each weight then
 * carries a relative error of at most 2^-9, so an output element moves by at
 * most 2^-9 max_j |v_j| (its keys' largest value component) more than with
 * the pair: within a 2e-2 bound while the values stay below 10 in magnitude
 * (N(0,1) values), not with large outlier channels.  The caller decides. */
#define LCCA_P_BF16 0x200

typedef struct {
    int32_t dtype;        /* lcca_dtype of the stored entries                    */
    int32_t dim;          /* elements per entry                                  */
    int32_t ratio_m;      /* tokens per entry; 256 % ratio_m == 0                */
    int32_t num_blocks;   /* physical blocks in the pool                         */
    void*   data;         /* device [num_blocks][256/ratio_m][row bytes]          */
    void*   scale;        /* device: MXFP4 u8 [..][dim/32]; FP8 float [..] or NULL */
} lcca_paged_cache;

typedef struct {
    int32_t dtype;        /* LCCA_F32, LCCA_BF16 or LCCA_FP8_E4M3                */
    int32_t dim;          /* elements per token (= the pool's dim)               */
    int32_t capacity;     /* slots per sequence (>= window; see the ring rule above) */
    int32_t window;       /* positions attended: max(0, p-window+1) .. p          */
    void*   data;         /* device [batch][capacity][row bytes]                 */
    float*  scale;        /* device [batch][capacity]; FP8 only                  */
} lcca_window_cache;

typedef struct {
    int32_t batch;              /* sequences                                     */
    int32_t max_blocks_per_seq; /* row stride of block_table                     */
    const int32_t* block_table; /* device [batch][max_blocks_per_seq]            */
} lcca_pages;

typedef struct {
    int32_t num_rows;           /* query rows                                    */
    int32_t max_pos;            /* host: upper bound of every row_pos (sizes grids) */
    const int32_t* row_seq;     /* device [num_rows] sequence of each row        */
    const int32_t* row_pos;     /* device [num_rows] position of each row        */
} lcca_rows;

/* The remainder ring's four arrays may be carved from one allocation of
 * lcca_remainder_bytes() bytes: kv at offset 0, then ik, kv_logit and ik_logit,
 * each starting at the previous array's end rounded up to 256 bytes (ik and
 * ik_logit are absent, 0 bytes, when ik_dim is 0).  Returns 0 for an invalid
 * argument (batch < 1, ratio_m not dividing 256, kv_dim < 1, ik_dim < 0, a
 * token dtype other than F32 or BF16). */
size_t lcca_remainder_bytes(int32_t batch, int32_t ratio_m, int32_t kv_dim, int32_t ik_dim, int32_t tok_dtype);

typedef struct {
    int32_t tok_dtype;          /* LCCA_F32 or LCCA_BF16 (the token dtype)       */
    void*   kv;                 /* device [batch][ratio_m][kv dim]               */
    void*   ik;                 /* device [batch][ratio_m][indexer dim] or NULL  */
    float*  kv_logit;           /* device [batch][ratio_m]                       */
    float*  ik_logit;           /* device [batch][ratio_m] or NULL               */
} lcca_remainder;

/*
 * lcca_compress_append -- fold new tokens into compressed entries and append.
 *
 * [P1 "Kako funkcionira optimizacija KV cachea?": the cache is compressed by
 * weighted summation of tokens, 4x (CSA) to 128x (HCA); P1 "Sto je vLLM morao
 * rijesiti u integraciji?": paged 256-position blocks, remainder as window
 * state.]  Sequence b receives n_b = cu_new[b+1] - cu_new[b] tokens at
 * positions start_pos[b] .. start_pos[b]+n_b-1 (rows cu_new[b].. of the token
 * arrays).  For each group g of ratio_m tokens completed by the chunk, and for
 * each stream (shared-KV vectors; indexer keys if `ik` is given):
 *     w_i = softmax_i(a_{g m + i})  over the group's per-token logits a,
 *     C_g = sum_i w_i x_{g m + i}   (fp32),
 * encoded to the pool dtype and stored as entry g.  Group tokens older than
 * the chunk are read from the remainder ring; new tokens of a still
 * incomplete group are stored into it.  The last min(n_b, capacity) new
 * tokens are encoded into the window ring (rows later attended inside the
 * chunk need capacity >= window + n_b - 1, see the window ring above).
 *   cu_new     device int32 [batch+1], cu_new[0] = 0, nondecreasing
 *   start_pos  device int32 [batch]
 *   total_new  host: cu_new[batch] (the grid has one block per new token)
 *   kv_tok     device [total_new][kv->dim] of tok_dtype (F32 or BF16)
 *   kv_logit   device float [total_new]
 *   ik_tok, ik_logit   device, as above with ik->dim; both NULL iff ik NULL
 *   kv         pool of dtype F32, BF16 or MXFP4 (dim % 32 == 0 for MXFP4)
 *   ik         pool of dtype F32, BF16 or FP8 (raw E4M3, scale NULL), or NULL
 *   win        window ring of the kv stream (dim = kv->dim), or NULL
 *   rem        remainder ring (tok_dtype must match)
 * Stored codes: bf16 and E4M3 round to nearest even (E4M3 saturates at
 * +-448); MXFP4 uses the OCP rule: X = floor(log2(max|x|)) - 2 per 32
 * elements, elements RNE to E2M1 after division by 2^X, saturating at +-6.
 * Chunks of one sequence must be appended in position order; calls for
 * distinct sequences may be combined freely.
 * Rebuilding the rings of one layer (pool entries kept, rings lost, as on a
 * prefix-cache hit): append the sequence's tokens again from the multiple of
 * ratio_m at or below P - win->window up to P - 1, P being the next position
 * to append.  Every group of that range is complete within it, so no
 * remainder slot is read; its entries are rewritten with the same codes,
 * and the window ring (positions P - window .. P - 1) and the remainder ring
 * end as after the uninterrupted history.  A replay starting inside a group
 * would form that group from the remainder ring's stale contents.
 */
lcca_status lcca_compress_append(void* stream, const lcca_pages* pages,
                                 const int32_t* cu_new, const int32_t* start_pos, int32_t total_new,
                                 int32_t tok_dtype, const void* kv_tok, const float* kv_logit,
                                 const void* ik_tok, const float* ik_logit,
                                 const lcca_paged_cache* kv, const lcca_paged_cache* ik,
                                 const lcca_window_cache* win, const lcca_remainder* rem);

/*
 * lcca_compress_append_gated -- lcca_compress_append with per-channel gates.
 *
 * [P1 "Kako funkcionira optimizacija KV cachea?": tokens are folded by
 * weighted summation; here every channel of a token carries its own
 * aggregation logit, the per-channel variant of the same weighted sum.]  For
 * each completed group g, stream and channel c:
 *     w_ic = softmax_i(a_{g m + i, c})  over the group's m tokens,
 *     C_gc = sum_i w_ic x_{g m + i, c}  (fp32),
 * with the same encode, pages, window ring and remainder ring as
 * lcca_compress_append.  With equal logits in every channel the entries
 * equal the per-token call's.  Arguments as lcca_compress_append, except:
 *   kv_logit   device float [total_new][kv->dim]
 *   ik_logit   device float [total_new][ik->dim] (NULL iff ik NULL)
 *   rem        its kv_logit is float [batch][ratio_m][kv->dim] and its
 *              ik_logit float [batch][ratio_m][ik->dim]: a ring slot holds
 *              the token's whole logit row
 * Token and logit arrays are read in 16-byte units: 16-byte aligned.
 * One workgroup per new token.
 */
lcca_status lcca_compress_append_gated(void* stream, const lcca_pages* pages,
                                       const int32_t* cu_new, const int32_t* start_pos, int32_t total_new,
                                       int32_t tok_dtype, const void* kv_tok, const float* kv_logit,
                                       const void* ik_tok, const float* ik_logit,
                                       const lcca_paged_cache* kv, const lcca_paged_cache* ik,
                                       const lcca_window_cache* win, const lcca_remainder* rem);

/*
 * lcca_index_logits -- sparse MQA logits of the indexer.
 *
 * [P3 "Vykon neprinesl jeden kernel": the indexer scores only candidate
 * positions.]  For row r (sequence b, position p) and every visible entry
 * g < n_r = floor((p+1)/m):
 *     logits[r*ld + g] = s_I * sum_h w_idx[r][h] * max(0, q_idx[r][h] . K_g)
 * with K_g the dequantised indexer key of entry g.  Entries g >= n_r are not
 * written.  fp32 accumulation; bf16 queries and bf16/FP8 keys use MFMA on
 * exactly upconverted keys.
 *   q_idx   device [num_rows][HI][ik->dim] of q_dtype (F32 with F32 keys;
 *           BF16 with BF16 or FP8 keys; BF16 | LCCA_Q_FP8 with FP8 keys
 *           quantises the query to FP8, see LCCA_Q_FP8)
 *   w_idx   device float [num_rows][HI]
 *   logits  device float [num_rows][ld], ld >= max visible entries
 * BF16 path: HI % 32 == 0 and ik->dim % 64 == 0 (HI <= 128, dim <= 256).
 */
lcca_status lcca_index_logits(void* stream, const lcca_pages* pages, const lcca_rows* rows,
                              int32_t q_dtype, const void* q_idx, int32_t HI, const float* w_idx, float s_I,
                              const lcca_paged_cache* ik, float* logits, int64_t ld);

/*
 * lcca_topk_select -- the entries each row attends to.
 *
 * [P1 "Kako funkcionira optimizacija KV cachea?": attention is restricted to
 * the top-k compressed tokens.]  topk_idx[r][0..] receives the min(k, n_r)
 * entries with the largest logits[r][g], g < n_r; equal logits rank the
 * smaller entry first (-0.0 equals +0.0).  The set is written in ascending
 * entry order and padded with -1 up to k.  NaN logits give an unspecified
 * selection.
 *   logits    device float [num_rows][ld]
 *   topk_idx  device int32 [num_rows][k]
 *   ws        device workspace of at least lcca_topk_workspace_size() bytes
 *             for the same rows, ratio_m and k, 16-byte aligned; may be NULL
 *             when that size is 0 (rows of at most 32,768 visible entries).
 *             Rows longer than that are selected in two launches: the top-k
 *             of each 16,384-entry slice, then the top-k of those
 *             candidates (the same set and order).  Too small a workspace
 *             returns LCCA_ERR_WORKSPACE.
 * Rows of more than 2^18 visible entries ((max_pos + 1) / ratio_m) return
 * LCCA_ERR_UNSUPPORTED (the selection keeps a bitmap of the row in LDS), and
 * so do rows over 32,768 entries whose slices' candidates (slices times k)
 * exceed 2^18: the candidates' selection keeps the same bitmap.
 */
size_t lcca_topk_workspace_size(const lcca_rows* rows, int32_t ratio_m, int32_t k);
lcca_status lcca_topk_select(void* stream, const lcca_rows* rows, int32_t ratio_m,
                             const float* logits, int64_t ld, int32_t k, int32_t* topk_idx,
                             void* ws, size_t ws_bytes);

/*
 * lcca_decode_select -- compress_append, index_logits and topk_select of a
 * decode step with one launch fewer.
 *
 * [P1 "Kako funkcionira optimizacija KV cachea?" and P3 "Vykon neprinesl
 * jeden kernel": the same three stages as above.]  Every sequence appends
 * exactly one token and queries at it: total_new == pages->batch ==
 * rows->num_rows, and for every b, cu_new[b] == b, row_seq[b] == b and
 * row_pos[b] == start_pos[b].  Launch 1 computes the logits of every row;
 * the entry a row's own token completes (not yet in the pool) is formed by
 * the kernel from the remainder ring and the token with compress_append's
 * arithmetic, so it is scored from exactly the codes the pool receives.
 * Launch 2 runs the top-k selection of every row and, beside it, the whole
 * of compress_append for the new tokens.  Pools, rings and the logits of
 * the entries already in the pool equal those of lcca_compress_append,
 * lcca_index_logits and lcca_topk_select called in that order; the logit of
 * the entry a row's token completes is summed in another order (within the
 * indexer's fp32 bound of theirs); the top-k lists are lcca_topk_select's on
 * these logits.  A row whose sequence does not
 * satisfy the device-side part of the contract (cu_new, start_pos) gets a
 * NaN logit for the entry its token completes.
 * The indexer launch also counts, per row, the logits whose order keys
 * share each leading 12-bit digit.  With rows of up to 32,768 visible
 * entries the selection starts from those counts instead of counting
 * itself.  Longer rows take three launches: a selection in each slice of
 * 16,384 entries, then the selection among the slices' candidates beside
 * compress_append; from the row's counts every slice knows the row's
 * boundary digit and how many entries the row takes from it, so it keeps
 * only its keys above that digit and the largest of its keys in it (at most
 * k, padded), a set that holds every entry of the row's top-k.
 * Arguments: those of the three calls, and
 *   ws   device workspace of at least lcca_decode_select_workspace_size()
 *        bytes for the same rows, ratio_m and k, 16-byte aligned: for rows
 *        over 32,768 entries first the slices' candidates (the size of
 *        lcca_topk_workspace_size), then the counts, uint32
 *        [num_rows][4096], which must be all zero before the first call on
 *        this workspace; every call leaves them zero (the selection clears
 *        them once read).
 * Supported: BF16 queries and tokens, an indexer pool, fewer than 64 rows,
 * ratio_m <= 4, ld % 4 == 0 and 16-byte aligned logits, and rows of at most
 * 32,768 visible entries or with at most 32,768 slice candidates (16,384-entry
 * slices times k); otherwise LCCA_ERR_UNSUPPORTED and nothing runs.
 */
lcca_status lcca_decode_select(void* stream, const lcca_pages* pages, const lcca_rows* rows,
                               const int32_t* cu_new, const int32_t* start_pos, int32_t total_new,
                               int32_t tok_dtype, const void* kv_tok, const float* kv_logit,
                               const void* ik_tok, const float* ik_logit,
                               const lcca_paged_cache* kv, const lcca_paged_cache* ik,
                               const lcca_window_cache* win, const lcca_remainder* rem,
                               int32_t q_dtype, const void* q_idx, int32_t HI, const float* w_idx, float s_I,
                               float* logits, int64_t ld, int32_t k, int32_t* topk_idx,
                               void* ws, size_t ws_bytes);
size_t lcca_decode_select_workspace_size(const lcca_rows* rows, int32_t ratio_m, int32_t k);

/*
 * lcca_sparse_attn_fwd -- attention over selected entries plus the window.
 *
 * [P1 "Kako funkcionira optimizacija KV cachea?": shared KV vectors, top-k
 * sparse attention over compressed tokens, and a local window of full
 * vectors.]  For row r (sequence b, position p) the keys are the dequantised
 * entries listed in topk_idx[r][0..k) (entries < 0 or >= n_r are skipped;
 * topk_idx NULL means every visible entry g < n_r), followed by the window
 * tokens max(0, p - win->window + 1) .. p (read from ring slots t % capacity,
 * so they must not have been overwritten since: see the window ring above).
 * One vector is key and value
 * (value = its first d_v elements).  For each head h:
 *     s_j = sm_scale * q[r][h] . k_j,
 *     out[r][h] = sum_j softmax(s)_j v_j,    lse[r][h] = ln sum_j exp(s_j)
 * with all keys in ONE softmax.  Keys are split across workgroups and the
 * partial softmax states are merged (max, rescaled sums); for BF16 outputs
 * a split's O / sum is kept as fp16 (11 significant bits against the
 * output's 8) with a power-of-two range scale per split, head and 4 value
 * dims, for F32 outputs in fp32.
 *   q        device [num_rows][H][kv->dim] of q_dtype (F32 with F32 cache;
 *            BF16 otherwise; BF16 | LCCA_Q_FP8 with an MXFP4 cache quantises
 *            it to FP8, see LCCA_Q_FP8; other combinations with the flag
 *            return LCCA_ERR_UNSUPPORTED; | LCCA_P_BF16: see there)
 *   out      device [num_rows][H][d_v] of out_dtype (F32 or BF16)
 *   lse      device float [num_rows][H] or NULL
 *   ws       device workspace of at least lcca_sparse_attn_workspace_size()
 *            bytes for the same arguments, 16-byte aligned (may be NULL if
 *            that size is 0)
 * BF16 path: kv dtype BF16 or MXFP4, window BF16 or FP8, H a multiple of 64
 * (64 heads per workgroup), (dim, d_v) in {(576, 576), (576, 512), (128, 128)};
 * an FP8 window's scale array must be given.  Other combinations return
 * LCCA_ERR_UNSUPPORTED.
 */
lcca_status lcca_sparse_attn_fwd(void* stream, const lcca_pages* pages, const lcca_rows* rows,
                                 int32_t q_dtype, const void* q, int32_t H, int32_t d_v, float sm_scale,
                                 const lcca_paged_cache* kv, const int32_t* topk_idx, int32_t k,
                                 const lcca_window_cache* win, int32_t out_dtype, void* out, float* lse,
                                 void* ws, size_t ws_bytes);

/* Workspace bytes lcca_sparse_attn_fwd needs for these arguments
 * (partial softmax states of the key splits). */
size_t lcca_sparse_attn_workspace_size(const lcca_rows* rows, int32_t ratio_m, int32_t H, int32_t dim,
                                       int32_t d_v, int32_t k, int32_t topk_given, int32_t window);

/*
 * lcca_sparse_attn_fwd_noalloc -- lcca_sparse_attn_fwd without a workspace.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops that must not call hipMalloc, harnesses that forbid
 * it.  Same arguments, results and kernels as lcca_sparse_attn_fwd; the split
 * partial states go to the library's own device scratch array of
 * LCCA_ATTN_SCRATCH_BYTES (64 MiB), one per GPU, held from the library's load
 * on that GPU until the process ends.  The call allocates nothing and frees
 * nothing.
 *   - A call whose partial states (lcca_sparse_attn_workspace_size for the
 *     same arguments) exceed LCCA_ATTN_SCRATCH_BYTES returns
 *     LCCA_ERR_UNSUPPORTED and launches nothing.
 *   - Every call on one GPU uses the same array: calls that overlap on one
 *     GPU (on different streams, or from different threads without ordering)
 *     race and give undefined results.  Calls ordered on one stream are safe.
 *     Nothing in the array needs clearing between calls.
 *   - The array's device address is looked up on the first call on each GPU
 *     (with that GPU current); a failure returns LCCA_ERR_HIP.
 */
#define LCCA_ATTN_SCRATCH_BYTES ((size_t)64 << 20)
lcca_status lcca_sparse_attn_fwd_noalloc(void* stream, const lcca_pages* pages, const lcca_rows* rows,
                                         int32_t q_dtype, const void* q, int32_t H, int32_t d_v, float sm_scale,
                                         const lcca_paged_cache* kv, const int32_t* topk_idx, int32_t k,
                                         const lcca_window_cache* win, int32_t out_dtype, void* out, float* lse);

/*
 * lcca_rope -- rotary position embedding of a slice of dims, in place.
 *
 * [P1 "Kako funkcionira optimizacija KV cachea?": the shared KV vectors are
 * used with RoPE and the inverse rotation is applied to the output.]  The
 * pages fix no convention, so the caller gives it.  For every row r, head h
 * and pair i < rope_dim / 2 of the slice [rope_off, rope_off + rope_dim) of
 * x[r][h], the pair (a, b) = dims (rope_off + 2i, rope_off + 2i + 1)
 * (interleaved, the default) or (rope_off + i, rope_off + i + rope_dim / 2)
 * (flag LCCA_ROPE_HALF) becomes
 *     (a cos t - b sin t, a sin t + b cos t),   t = fp32(pos[r]) * f_i
 * (an fp32 product; t negated with flag LCCA_ROPE_INVERSE, which undoes the
 * forward rotation at the same positions).  f_i = inv_freq[i] if inv_freq
 * is given (host float [rope_dim / 2], e.g. a scaled table), else
 * fp32(theta^(-2i / rope_dim)) formed in double.  cos/sin and the rotation
 * are fp32; BF16 results are rounded to nearest even.  Dims outside the slice
 * are not touched.  Use: queries and new tokens before they are scored or
 * compressed (rows = tokens, heads = 1 for the shared vectors), and the
 * inverse on the attention output at the query positions.
 *   dtype     LCCA_F32 or LCCA_BF16 (else LCCA_ERR_UNSUPPORTED)
 *   x         device [rows][heads][dim] of dtype, read and written
 *   pos       device int32 [rows] (any value)
 *   rope_dim  even, 2..256, with rope_off >= 0 and rope_off + rope_dim <= dim
 *   flags     LCCA_ROPE_HALF | LCCA_ROPE_INVERSE (other bits: invalid)
 * rows == 0 launches nothing.  Vector loads are used when x is 16-byte
 * aligned and rope_off, rope_dim and dim are multiples of 8.
 */
#define LCCA_ROPE_HALF    1
#define LCCA_ROPE_INVERSE 2
lcca_status lcca_rope(void* stream, int32_t dtype, void* x, int64_t rows, int32_t heads, int32_t dim,
                      int32_t rope_off, int32_t rope_dim, const int32_t* pos, double theta, const float* inv_freq,
                      int32_t flags);

/*
 * lcca_debug_check -- index violations the debug library's kernels found.
 *
 * For development and for callers that cannot vouch for their device-side
 * indices.  In the debug library (liblcca_debug.so: every kernel built with
 * LCCA_DEBUG, the same entry points and results for valid inputs) each
 * block-table entry, row_seq, row_pos, cu_new and start_pos value a kernel
 * reads is checked before it forms an address.  A value outside its range
 * (LCCA_DBG_* above) is replaced by the range's first value (block 0,
 * sequence 0, position 0; a compress_append token of a bad chunk is treated
 * as a chunk of its own at position 0), so every access stays inside the
 * caller's buffers and every kernel finishes; the outputs of such a call are
 * unspecified, and the violation's bit is set in the current device's error
 * word.  lcca_debug_check waits for `stream`, reads the word into *bits (may
 * be NULL) and clears it.  Returns LCCA_OK if no bit was set,
 * LCCA_ERR_DEVICE_INDEX (with the bits named in lcca_last_error()) if one
 * was, LCCA_ERR_HIP if a runtime call failed.  The word is shared by every
 * stream of the device: calls on other streams that run meanwhile add their
 * bits.  The release library keeps no word: there it sets *bits = 0 and
 * returns LCCA_ERR_UNSUPPORTED.
 */
lcca_status lcca_debug_check(void* stream, uint32_t* bits);

const char* lcca_status_string(lcca_status s);
const char* lcca_last_error(void);
const char* lcca_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LCCA_H */
