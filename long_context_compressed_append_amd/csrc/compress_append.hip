// compress_append kernels; the per-slice device code is in compress_dev.h.
// [Page "vLLM uveo DeepSeek V4 s 8,7x manjim KV cacheom", section "Kako
//  funkcionira optimizacija KV cachea?": weighted summation of tokens;
//  section "Sto je vLLM morao rijesiti u integraciji?": 256-position blocks,
//  remainder of the compressor kept as sliding-window state.]
//
// Two launch shapes:
//   * few new tokens (decode) or groups of more than 32 tokens: grid (new
//     token, slice) of compress_dev.h;
//   * chunks (chunked prefill): one workgroup per 16 consecutive new tokens
//     (counted over the whole call), which writes their window slots, forms
//     every group one of them completes (both streams, all dimensions) and,
//     for the sequence it is assigned to, the remainder ring.  The entries'
//     arithmetic is the slice kernel's, step for step (weights by one wave's
//     max, exponentials and butterfly sum; products w_i x_i rounded one by one
//     and summed in token order), so both shapes store the same codes.
#include "compress_dev.h"

namespace lcca {

namespace {

template <int TOK>
__global__ __launch_bounds__(cmp::kThreads) void compress_append_kernel(CompressArgs p) {
    cmp::compress_append_body<TOK>(p, blockIdx.x, blockIdx.y);
}

constexpr int kChunkTokens = 16;            // new tokens per workgroup
constexpr int kChunkMaxM = 8;               // largest group the chunk kernel forms
constexpr int kChunkMinTokens = 64;         // calls with fewer new tokens use the slice grid
constexpr int kRoundSlots = 4;              // 8-dimension items per thread per round of loads
constexpr int kWinSlots = 5;                // window items per thread requested with the first round

// The encode of one 8-dimension chunk of an entry (v: its aggregate values)
// into the pool; MXFP4 blocks of 32 dimensions are held by four adjacent
// lanes (amax over them by two lane exchanges, the scale byte by the first).
__device__ __forceinline__ void store_entry_chunk(const CompressArgs& p, bool ik, int64_t row, int d0, const float (&v)[8],
                                                  bool active) {
    const int dim = ik ? p.dI : p.D;
    const int dt = ik ? p.ik_dtype : p.kv_dtype;
    uint8_t* data = reinterpret_cast<uint8_t*>(ik ? p.ik_data : p.kv_data);
    if (dt == DT_MXFP4) {
        // (every lane takes part in the exchanges; inactive lanes hold zeros)
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(v[e]));
        a = fmaxf(a, lane_xor<1>(a));
        a = fmaxf(a, lane_xor<2>(a));
        const int X = mx_scale_exp(a);
        uint32_t wd = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) wd |= fp4_code(ldexpf(v[e], -X)) << (4 * e);
        if (active) {
            *reinterpret_cast<uint32_t*>(data + row * (int64_t)(dim / 2) + d0 / 2) = wd;
            if ((d0 & 31) == 0) reinterpret_cast<uint8_t*>(p.kv_scale)[row * (int64_t)(dim / 32) + d0 / 32] = (uint8_t)(X + 127);
        }
        return;
    }
    if (!active) return;
    if (dt == DT_BF16) {
        uint16_t* o = reinterpret_cast<uint16_t*>(data) + row * dim + d0;
        *reinterpret_cast<u32x4*>(o) = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                                             pack_bf16x2(v[6], v[7])};
    } else if (dt == DT_FP8) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            lo |= f32_to_fp8(v[e]) << (8 * e);
            hi |= f32_to_fp8(v[4 + e]) << (8 * e);
        }
        *reinterpret_cast<u32x2*>(data + row * (int64_t)dim + d0) = u32x2{lo, hi};
    } else {
        float* o = reinterpret_cast<float*>(data) + row * dim + d0;
        *reinterpret_cast<f32x4*>(o) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(o + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
}

// One 8-value chunk of a token into its window slot (F32, BF16, or FP8 with
// the token's scale `sc`).
__device__ __forceinline__ void store_window_chunk(const CompressArgs& p, int64_t slot, int d0, const float (&x)[8],
                                                   float sc) {
    const int D = p.D;
    uint8_t* wd = reinterpret_cast<uint8_t*>(p.win_data);
    if (p.win_dtype == DT_FP8) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            lo |= f32_to_fp8(x[e] / sc) << (8 * e);
            hi |= f32_to_fp8(x[4 + e] / sc) << (8 * e);
        }
        *reinterpret_cast<u32x2*>(wd + slot * D + d0) = u32x2{lo, hi};
    } else if (p.win_dtype == DT_BF16) {
        *reinterpret_cast<u32x4*>(wd + (slot * D + d0) * 2) =
            u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
    } else {
        float* o = reinterpret_cast<float*>(wd) + slot * D + d0;
        *reinterpret_cast<f32x4*>(o) = f32x4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<f32x4*>(o + 4) = f32x4{x[4], x[5], x[6], x[7]};
    }
}

template <int TOK>
__global__ __launch_bounds__(cmp::kThreads) void compress_chunk_kernel(CompressArgs p, int total_new) {
    constexpr int NT = cmp::kThreads;
    __shared__ int cu_lds[cmp::kSeqLds + 1], sp_lds[cmp::kSeqLds];
    __shared__ int tk_b[kChunkTokens], tk_pos[kChunkTokens], tk_start[kChunkTokens], tk_end[kChunkTokens];
    __shared__ long long tk_c0[kChunkTokens];
    __shared__ int grp_tok[kChunkTokens], n_grp;
    __shared__ unsigned int tail_mask;         // tokens that carry their sequence's remainder-ring duty
    __shared__ long long grp_row[kChunkTokens];
    __shared__ float w_lds[2][kChunkTokens][kChunkMaxM];
    __shared__ unsigned int amax_lds[kChunkTokens];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = (int)blockIdx.x * kChunkTokens;
    const int ntok = min(kChunkTokens, total_new - t0);
    const int m = p.m;
    const bool in_lds = p.batch <= cmp::kSeqLds;
    if (in_lds) {
        for (int i = tid; i <= p.batch; i += NT) {
            cu_lds[i] = p.cu_new[i];
            if (i < p.batch) sp_lds[i] = p.start_pos[i];
        }
    }
    if (tid == 0) { n_grp = 0; tail_mask = 0u; }
    if (tid < kChunkTokens) amax_lds[tid] = 0u;
    __syncthreads();
    // each token: its sequence, position, and whether it completes a group
    // or carries the sequence's remainder-ring duty.  The pool row of a group
    // it completes is requested here and written to LDS only after the
    // weights are formed, so nothing waits for the block table meanwhile.
    int my_grp = -1, my_blk = 0, my_slot = 0;
    if (tid < ntok) {
        const int t = t0 + tid;
        auto cu = [&](int i) { return in_lds ? cu_lds[i] : p.cu_new[i]; };
        int lo = 0, hi = p.batch - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cu(mid) <= t) lo = mid; else hi = mid - 1;
        }
        int c0 = cu(lo), n = cu(lo + 1) - c0;
        int start = in_lds ? sp_lds[lo] : p.start_pos[lo];
        if (chunk_invalid(t, c0, c0 + n, start, p.total_new, p.max_blocks, p.dbg, kDbgChunk)) {
            c0 = t; n = 1; start = 0;             // (debug builds) a chunk of this token alone at position 0
        }
        const int end = start + n, pos = start + (t - c0);
        tk_b[tid] = lo; tk_pos[tid] = pos; tk_start[tid] = start; tk_end[tid] = end; tk_c0[tid] = c0;
        const int g0 = start / m;
        // the chunk reads ring slots (its first group starts before it) and
        // rewrites ring slots (it ends inside a group): the tail waits for the
        // first group's reads, in the workgroup that forms it
        const bool race = (start % m) != 0 && (end % m) != 0 && end >= (g0 + 1) * m;
        const bool tail_here = (end % m) != 0 && (race ? pos == (g0 + 1) * m - 1 : pos == end - 1);
        if (tail_here) atomicOr(&tail_mask, 1u << tid);
        if ((pos + 1) % m == 0) {
            const int k = atomicAdd(&n_grp, 1);
            grp_tok[k] = tid;
            const int g = pos / m, E = 256 / m;
            my_grp = k;
            my_blk = p.block_table[(int64_t)lo * p.max_blocks + g / E];
            my_slot = g % E;
        }
    }
    __syncthreads();
    const int ng = n_grp;
    // Every load of the workgroup's first round goes out before anything is
    // formed: the window slots' tokens (bf16 / fp32 windows; kWinSlots items
    // per thread) and the entries' token chunks, then the group weights'
    // logits, so their latencies overlap.
    const int nch = p.D / 8;
    const int witems = p.win_data != nullptr ? ntok * nch : 0;
    const bool win_pre = p.win_data != nullptr && p.win_dtype != DT_FP8;
    cmp::RawChunk<TOK> wraw[kWinSlots];
    const int win_cap = p.win_cap;
    auto win_item_live = [&](int it) __attribute__((always_inline)) {
        return it < witems && tk_pos[it / nch] >= tk_end[it / nch] - win_cap;
    };
    if (win_pre) {
#pragma unroll
        for (int j = 0; j < kWinSlots; ++j) {
            const int it = tid + NT * j;
            if (win_item_live(it)) cmp::load_chunk<TOK>(p.kv_tok, (int64_t)(t0 + it / nch) * p.D + 8 * (it % nch), wraw[j]);
        }
    }
    // entries: items (group, stream, 8-dimension chunk), SLOTS per thread per
    // round; a round requests all of its tokens' chunks before forming any.
    // A group's items are padded to a multiple of four, and MXFP4 pools (kv
    // only) have dimensions in multiples of 32, so the four chunks of an MXFP4
    // block sit on four adjacent lanes.
    constexpr int SLOTS = TOK == DT_F32 ? kRoundSlots / 2 : kRoundSlots;
    const int nkv = p.D / 8, nik = p.ik_data != nullptr ? p.dI / 8 : 0;
    const int per = nkv + ((nik + 3) & ~3);
    const int items = ng * per;
    cmp::RawChunk<TOK> raw[SLOTS][kChunkMaxM];
    auto load_round = [&](int base) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < SLOTS; ++j) {
            const int it = base + tid + NT * j;
            if (it < items && it % per < nkv + nik) {
                const int k = it / per, u = it % per, tk = grp_tok[k];
                const bool ik = u >= nkv;
                const int d0 = ik ? (u - nkv) * 8 : u * 8, dim = ik ? p.dI : p.D;
                const int b = tk_b[tk], start = tk_start[tk], g = tk_pos[tk] / m;
                const void* tok = ik ? p.ik_tok : p.kv_tok;
                const void* rtok = ik ? p.rem_ik : p.rem_kv;
#pragma unroll
                for (int i = 0; i < kChunkMaxM; ++i) {
                    if (i < m) {
                        const int t = g * m + i;
                        const int64_t trow = t >= start ? tk_c0[tk] + (t - start) : (int64_t)b * m + t % m;
                        cmp::load_chunk<TOK>(t >= start ? tok : rtok, trow * dim + d0, raw[j][i]);
                    }
                }
            }
        }
    };
    auto form_round = [&](int base) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < SLOTS; ++j) {
            const int it = base + tid + NT * j;
            const bool active = it < items && it % per < nkv + nik;
            const int k = active ? it / per : 0, u = active ? it % per : 0;
            const bool ik = u >= nkv;
            const int d0 = ik ? (u - nkv) * 8 : u * 8;
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.0f;
            if (active) {
                // the products rounded one by one, then summed in token
                // order, as in the slice kernel
#pragma clang fp contract(off)
                const float* w = &w_lds[ik ? 1 : 0][k][0];
#pragma unroll
                for (int i = 0; i < kChunkMaxM; ++i) {
                    if (i < m) {
                        float x[8];
                        cmp::unpack_chunk<TOK>(raw[j][i], x);
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] = v[e] + fmaf(w[i], x[e], 0.0f);
                    }
                }
            }
            // MXFP4 lane exchanges: every lane of the wave takes part
            store_entry_chunk(p, ik, active ? grp_row[k] : 0, d0, v, active);
        }
    };
    load_round(0);
    // softmax weights of each group's logits, one wave per (group, stream),
    // with the slice kernel's reductions
    const int nstream = p.ik_data != nullptr ? 2 : 1;
    for (int it = wave; it < ng * nstream; it += NT / 64) {
        const int k = it / nstream, s = it % nstream;
        const int tk = grp_tok[k];
        const int b = tk_b[tk], start = tk_start[tk], g = tk_pos[tk] / m;
        const float* lg = s ? p.ik_logit : p.kv_logit;
        const float* rlg = s ? p.rem_ik_logit : p.rem_kv_logit;
        float a = -INFINITY;
        if (lane < m) {
            const int t = g * m + lane;
            a = t >= start ? lg[tk_c0[tk] + (t - start)] : rlg[(int64_t)b * m + t % m];
        }
        const float mx = wave_max(a);
        const float e = lane < m ? expf(a - mx) : 0.0f;
        const float sum = wave_sum(e);
        if (lane < m) w_lds[s][k][lane] = e / sum;
    }
    if (my_grp >= 0)
        grp_row[my_grp] = (long long)checked(my_blk, 0, p.n_blocks - 1, p.dbg, kDbgBlock) * (256 / m) + my_slot;
    __syncthreads();
    form_round(0);
    for (int base = NT * SLOTS; base < items; base += NT * SLOTS) {
        load_round(base);
        form_round(base);
    }
    // window slots of the tokens among the last `capacity` of their chunk:
    // items (token, 8-value chunk).  bf16 / fp32 windows: the prefetched
    // items, then any further rounds.  FP8 windows take each token's max
    // first (a pass of loads and an LDS max), then encode in a second pass.
    if (win_pre) {
#pragma unroll
        for (int j = 0; j < kWinSlots; ++j) {
            const int it = tid + NT * j;
            if (!win_item_live(it)) continue;
            const int tk = it / nch, c = it % nch;
            float x[8];
            cmp::unpack_chunk<TOK>(wraw[j], x);
            store_window_chunk(p, (int64_t)tk_b[tk] * p.win_cap + tk_pos[tk] % p.win_cap, 8 * c, x, 1.0f);
        }
    }
    if (p.win_data != nullptr) {
        const bool fp8 = p.win_dtype == DT_FP8;
        const int first = win_pre ? NT * kWinSlots : 0;
        for (int pass = fp8 ? 0 : 1; pass < 2; ++pass) {
            if (pass == 1 && fp8) __syncthreads();
            for (int base = first; base < witems; base += NT * kRoundSlots) {
                cmp::RawChunk<TOK> rw[kRoundSlots];
#pragma unroll
                for (int j = 0; j < kRoundSlots; ++j) {
                    const int it = base + tid + NT * j;
                    if (win_item_live(it))
                        cmp::load_chunk<TOK>(p.kv_tok, (int64_t)(t0 + it / nch) * p.D + 8 * (it % nch), rw[j]);
                }
#pragma unroll
                for (int j = 0; j < kRoundSlots; ++j) {
                    const int it = base + tid + NT * j;
                    if (!win_item_live(it)) continue;
                    const int tk = it / nch, c = it % nch;
                    const int pos = tk_pos[tk];
                    float x[8];
                    cmp::unpack_chunk<TOK>(rw[j], x);
                    if (pass == 0) {
                        float a = 0.0f;
#pragma unroll
                        for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(x[e]));
                        atomicMax(&amax_lds[tk], __float_as_uint(a));      // non-negative: ordered as integers
                    } else {
                        float sc = 1.0f;
                        const int64_t slot = (int64_t)tk_b[tk] * p.win_cap + pos % p.win_cap;
                        if (fp8) {
                            const float amax = __uint_as_float(amax_lds[tk]);
                            sc = amax > 0.0f ? amax / 448.0f : 1.0f;
                            if (c == 0) p.win_scale[slot] = sc;
                        }
                        store_window_chunk(p, slot, 8 * c, x, sc);
                    }
                }
            }
        }
    }
    // remainder rings of the sequences this workgroup carries the duty for
    // (several short chunks may end in one workgroup): after every read of
    // the rings above
    __syncthreads();
    for (unsigned int mask = tail_mask; mask != 0u; mask &= mask - 1u) {
        const int tk = __builtin_ctz(mask);
        const cmp::SeqChunk q{tk_b[tk], tk_start[tk], tk_end[tk], tk_end[tk] - tk_start[tk], tk_c0[tk]};
        const int tail0 = max((q.end / m) * m, q.start);
        for (int tt = tail0; tt < q.end; ++tt) cmp::write_ring<TOK>(p, q, tt);
    }
}

// ---------------------------------------------------------------------------
// Per-channel-gated groups
// ---------------------------------------------------------------------------
// Every channel of every token carries its own logit and the group's softmax
// is taken per channel: w_ic = exp(a_ic - max_j a_jc) / sum_j exp(a_jc - ...),
// C_c = sum_i w_ic x_ic.  One workgroup of kGatedThreads per new token; its
// threads cover the token's 8-channel chunks (both streams, an MXFP4 block's
// four chunks on four adjacent lanes) and, if the token completes a group,
// form that group's chunks: the channel maxima, the exponentials and their
// sum, then the weighted sum, in token order; then the pool dtype's encode.
// The window slot and the remainder ring (tokens and their logit rows) are
// written as in the per-token kernels, including the ordering of a chunk
// whose first group reads ring slots its tail rewrites.
constexpr int kGatedThreads = 128;

// One 8-channel chunk of group g of a stream: x from the token arrays (or the
// ring for tokens before the chunk), logits from the [n][dim] rows (or the
// ring's [batch*m][dim] rows).
template <int TOK>
__device__ __forceinline__ void gated_chunk(const CompressArgs& p, const cmp::SeqChunk& q, int g, bool ik, int d0,
                                            float (&v)[8]) {
    const int m = p.m, dim = ik ? p.dI : p.D;
    const void* tok = ik ? p.ik_tok : p.kv_tok;
    const void* rtok = ik ? p.rem_ik : p.rem_kv;
    const float* lg = ik ? p.ik_logit : p.kv_logit;
    const float* rlg = ik ? p.rem_ik_logit : p.rem_kv_logit;
    auto row_of = [&](int i, bool& fresh) -> int64_t {
        const int t = g * m + i;
        fresh = t >= q.start;
        return fresh ? q.c0 + (t - q.start) : (int64_t)q.b * m + t % m;
    };
    auto logits = [&](int i, float (&a)[8]) {
        bool fresh;
        const int64_t r = row_of(i, fresh);
        const f32x4* src = reinterpret_cast<const f32x4*>((fresh ? lg : rlg) + r * dim + d0);
        const f32x4 lo = src[0], hi = src[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) { a[e] = lo[e]; a[4 + e] = hi[e]; }
    };
    float mx[8], sum[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { mx[e] = -INFINITY; sum[e] = 0.0f; v[e] = 0.0f; }
    for (int i = 0; i < m; ++i) {
        float a[8];
        logits(i, a);
#pragma unroll
        for (int e = 0; e < 8; ++e) mx[e] = fmaxf(mx[e], a[e]);
    }
    for (int i = 0; i < m; ++i) {
        float a[8];
        logits(i, a);
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[e] += expf(a[e] - mx[e]);
    }
    for (int i = 0; i < m; ++i) {
        float a[8], x[8];
        logits(i, a);
        bool fresh;
        const int64_t r = row_of(i, fresh);
        cmp::RawChunk<TOK> raw;
        cmp::load_chunk<TOK>(fresh ? tok : rtok, r * dim + d0, raw);
        cmp::unpack_chunk<TOK>(raw, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = fmaf(expf(a[e] - mx[e]) / sum[e], x[e], v[e]);
    }
}

// Token tt of the chunk into its remainder-ring slot: the token's vectors and
// logit rows of both streams (16-byte units, all NT threads of the workgroup).
template <int TOK, int NT = kGatedThreads>
__device__ void write_ring_gated(const CompressArgs& p, const cmp::SeqChunk& q, int tt) {
    constexpr int esz = TOK == DT_F32 ? 4 : 2;
    const int64_t src = q.c0 + (tt - q.start);
    const int64_t slot = (int64_t)q.b * p.m + tt % p.m;
    auto copy = [&](const void* s, void* d, int64_t bytes_per_row) {
        const u32x4* s4 = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(s) + src * bytes_per_row);
        u32x4* d4 = reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(d) + slot * bytes_per_row);
        for (int i = threadIdx.x; i < bytes_per_row / 16; i += NT) d4[i] = s4[i];
    };
    copy(p.kv_tok, p.rem_kv, (int64_t)p.D * esz);
    copy(p.kv_logit, p.rem_kv_logit, (int64_t)p.D * 4);
    if (p.ik_data != nullptr) {
        copy(p.ik_tok, p.rem_ik, (int64_t)p.dI * esz);
        copy(p.ik_logit, p.rem_ik_logit, (int64_t)p.dI * 4);
    }
}

template <int TOK>
__global__ __launch_bounds__(kGatedThreads) void compress_gated_kernel(CompressArgs p) {
    constexpr int NT = kGatedThreads;
    constexpr int kWinChunks = 2048 / 8 / NT;            // kv dims <= 2048
    __shared__ int cu_lds[cmp::kSeqLds + 1], sp_lds[cmp::kSeqLds];
    __shared__ unsigned int amax_lds;
    const int t = (int)blockIdx.x, tid = threadIdx.x;
    if (tid == 0) amax_lds = 0u;
    __syncthreads();
    const cmp::SeqChunk q = cmp::seq_of<NT>(p, t, cu_lds, sp_lds);
    const int m = p.m;
    const int pos = q.start + (t - (int)q.c0);
    const int g0 = q.start / m;
    const bool race = (q.start % m) != 0 && (q.end % m) != 0 && q.end >= (g0 + 1) * m;
    const int tail0 = max((q.end / m) * m, q.start);
    const int nkv = p.D / 8, nik = p.ik_data != nullptr ? p.dI / 8 : 0;
    const int per = nkv + ((nik + 3) & ~3);

    // (1) the group this token completes
    if ((pos + 1) % m == 0) {
        const int g = pos / m, E = 256 / m;
        const int64_t row =
            (int64_t)checked(p.block_table[(int64_t)q.b * p.max_blocks + g / E], 0, p.n_blocks - 1, p.dbg, kDbgBlock) * E +
            g % E;
        for (int base = 0; base < per; base += NT) {
            const int u = base + tid;
            const bool active = u < per && u - nkv < nik;
            const bool ik = u >= nkv;
            const int d0 = ik ? (u - nkv) * 8 : u * 8;
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.0f;
            if (active) gated_chunk<TOK>(p, q, g, ik, d0, v);
            store_entry_chunk(p, ik, row, d0, v, active);
        }
        if (race && g == g0) {
            // this workgroup read the ring slots the chunk's tail rewrites
            __syncthreads();
            for (int tt = tail0; tt < q.end; ++tt) write_ring_gated<TOK>(p, q, tt);
        }
    }
    // (2) window slot
    if (p.win_data != nullptr && pos >= q.end - p.win_cap) {
        const int64_t slot = (int64_t)q.b * p.win_cap + pos % p.win_cap;
        float x[kWinChunks][8];
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < kWinChunks; ++j) {
            const int c = tid + NT * j;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[j][e] = 0.0f;
            if (c < nkv) {
                cmp::RawChunk<TOK> raw;
                cmp::load_chunk<TOK>(p.kv_tok, (int64_t)t * p.D + 8 * c, raw);
                cmp::unpack_chunk<TOK>(raw, x[j]);
#pragma unroll
                for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(x[j][e]));
            }
        }
        float sc = 1.0f;
        if (p.win_dtype == DT_FP8) {
            atomicMax(&amax_lds, __float_as_uint(a));        // non-negative: ordered as integers
            __syncthreads();
            const float amax = __uint_as_float(amax_lds);
            sc = amax > 0.0f ? amax / 448.0f : 1.0f;
            if (tid == 0) p.win_scale[slot] = sc;
        }
#pragma unroll
        for (int j = 0; j < kWinChunks; ++j) {
            const int c = tid + NT * j;
            if (c < nkv) store_window_chunk(p, slot, 8 * c, x[j], sc);
        }
    }
    // (3) remainder ring: the token itself if it is in the incomplete tail
    if (!race && pos >= tail0) write_ring_gated<TOK>(p, q, pos);
}

// Groups of more than kChunkMaxM tokens (decode with m = 128): the grid of
// the per-token slice kernel, (new token, 64-dimension slice), 256 threads =
// 32 token lanes x 8 chunks of 8 dimensions.  Each lane holds the logit and
// token chunks of tokens lane, lane + 32, ...; the channel maxima, the sums
// of exponentials and the weighted sums are each reduced over the lanes in
// LDS; wave 0 then encodes the slice's 64 dimensions (one per thread).
template <int TOK>
__device__ void gated_slice(const CompressArgs& p, const cmp::SeqChunk& q, int g, bool ik, int d0, float* red,
                            float* stat) {
    constexpr int LANES = cmp::kLanes, SD = cmp::kSliceDims, TPL = cmp::kMaxTokPerLane;
    const int m = p.m, dim = ik ? p.dI : p.D;
    const int tid = threadIdx.x, lane = tid / (SD / 8), ch = tid % (SD / 8);
    const int d = d0 + ch * 8;
    const bool active = d < dim;
    const void* tok = ik ? p.ik_tok : p.kv_tok;
    const void* rtok = ik ? p.rem_ik : p.rem_kv;
    const float* lg = ik ? p.ik_logit : p.kv_logit;
    const float* rlg = ik ? p.rem_ik_logit : p.rem_kv_logit;
    cmp::RawChunk<TOK> raw[TPL];
    float a[TPL][8];
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
        const int i = lane + LANES * j;
#pragma unroll
        for (int e = 0; e < 8; ++e) a[j][e] = -INFINITY;
        if (active && i < m) {
            const int t = g * m + i;
            const bool fresh = t >= q.start;
            const int64_t r = fresh ? q.c0 + (t - q.start) : (int64_t)q.b * m + t % m;
            cmp::load_chunk<TOK>(fresh ? tok : rtok, r * dim + d, raw[j]);
            const f32x4* src = reinterpret_cast<const f32x4*>((fresh ? lg : rlg) + r * dim + d);
            const f32x4 lo = src[0], hi = src[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) { a[j][e] = lo[e]; a[j][4 + e] = hi[e]; }
        }
    }
    // one per-channel reduction over the token lanes: red[lane][64] -> stat[64]
    auto reduce = [&](const float (&v)[8], bool is_max, float (&out)[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) red[lane * SD + ch * 8 + e] = v[e];
        __syncthreads();
        if (tid < SD) {
            float r = red[tid];
            for (int l = 1; l < LANES; ++l) r = is_max ? fmaxf(r, red[l * SD + tid]) : r + red[l * SD + tid];
            stat[tid] = r;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = stat[ch * 8 + e];
        __syncthreads();
    };
    float mx[8], sum[8], v[8], loc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        loc[e] = -INFINITY;
#pragma unroll
        for (int j = 0; j < TPL; ++j) loc[e] = fmaxf(loc[e], a[j][e]);
    }
    reduce(loc, true, mx);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        loc[e] = 0.0f;
#pragma unroll
        for (int j = 0; j < TPL; ++j)
            if (lane + LANES * j < m) loc[e] += expf(a[j][e] - mx[e]);
    }
    reduce(loc, false, sum);
#pragma unroll
    for (int e = 0; e < 8; ++e) loc[e] = 0.0f;
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
        if (active && lane + LANES * j < m) {
            float x[8];
            cmp::unpack_chunk<TOK>(raw[j], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) loc[e] = fmaf(expf(a[j][e] - mx[e]) / sum[e], x[e], loc[e]);
        }
    }
    reduce(loc, false, v);
    // wave 0: dimension d0 + tid of the slice
    if (tid < SD) {
        const int E = 256 / m;
        const int64_t row =
            (int64_t)checked(p.block_table[(int64_t)q.b * p.max_blocks + g / E], 0, p.n_blocks - 1, p.dbg, kDbgBlock) * E +
            g % E;
        cmp::store_slice_dim(p, ik, row, d0 + tid, stat[tid]);
    }
    __syncthreads();
    (void)v;
}

template <int TOK>
__global__ __launch_bounds__(cmp::kThreads) void compress_gated_slice_kernel(CompressArgs p) {
    __shared__ float red[cmp::kLanes * cmp::kSliceDims];
    __shared__ float stat[cmp::kSliceDims];
    __shared__ int cu_lds[cmp::kSeqLds + 1], sp_lds[cmp::kSeqLds];
    const int t = (int)blockIdx.x, s = (int)blockIdx.y;
    const cmp::SeqChunk q = cmp::seq_of(p, t, cu_lds, sp_lds);
    const int m = p.m;
    const int pos = q.start + (t - (int)q.c0);
    const int SK = (p.D + cmp::kSliceDims - 1) / cmp::kSliceDims;
    const int SI = p.ik_data != nullptr ? (p.dI + cmp::kSliceDims - 1) / cmp::kSliceDims : 0;
    const int g0 = q.start / m;
    const bool race = (q.start % m) != 0 && (q.end % m) != 0 && q.end >= (g0 + 1) * m;
    const int tail0 = max((q.end / m) * m, q.start);
    if (s == SK + SI) {
        cmp::write_window<TOK>(p, q, t, pos, red);
        if (!race && pos >= tail0) write_ring_gated<TOK, cmp::kThreads>(p, q, pos);
        return;
    }
    if ((pos + 1) % m == 0) {
        const int g = pos / m;
        if (race && g == g0) {
            // the whole first group here (it reads ring slots the tail rewrites),
            // then the tail
            if (s == 0) {
                for (int k = 0; k < SK; ++k) gated_slice<TOK>(p, q, g, false, k * cmp::kSliceDims, red, stat);
                for (int k = 0; k < SI; ++k) gated_slice<TOK>(p, q, g, true, k * cmp::kSliceDims, red, stat);
                for (int tt = tail0; tt < q.end; ++tt) write_ring_gated<TOK, cmp::kThreads>(p, q, tt);
            }
        } else {
            const bool ik = s >= SK;
            gated_slice<TOK>(p, q, g, ik, (ik ? s - SK : s) * cmp::kSliceDims, red, stat);
        }
    }
}

}  // namespace

hipError_t launch_compress_append(const CompressArgs& a, int total_new, hipStream_t stream) {
    if (total_new <= 0) return hipSuccess;
    if (total_new >= kChunkMinTokens && a.m <= kChunkMaxM) {
        const dim3 grid((total_new + kChunkTokens - 1) / kChunkTokens);
        if (a.tok_dtype == DT_F32)
            hipLaunchKernelGGL(compress_chunk_kernel<DT_F32>, grid, dim3(cmp::kThreads), 0, stream, a, total_new);
        else
            hipLaunchKernelGGL(compress_chunk_kernel<DT_BF16>, grid, dim3(cmp::kThreads), 0, stream, a, total_new);
        return hipGetLastError();
    }
    const int SK = (a.D + cmp::kSliceDims - 1) / cmp::kSliceDims;
    const int SI = a.ik_data != nullptr ? (a.dI + cmp::kSliceDims - 1) / cmp::kSliceDims : 0;
    dim3 grid(total_new, SK + SI + 1);
    if (a.tok_dtype == DT_F32)
        hipLaunchKernelGGL(compress_append_kernel<DT_F32>, grid, dim3(cmp::kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(compress_append_kernel<DT_BF16>, grid, dim3(cmp::kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_compress_gated(const CompressArgs& a, int total_new, hipStream_t stream) {
    if (total_new <= 0) return hipSuccess;
    if (a.m > kChunkMaxM) {
        const int SK = (a.D + cmp::kSliceDims - 1) / cmp::kSliceDims;
        const int SI = a.ik_data != nullptr ? (a.dI + cmp::kSliceDims - 1) / cmp::kSliceDims : 0;
        const dim3 grid(total_new, SK + SI + 1);
        if (a.tok_dtype == DT_F32)
            hipLaunchKernelGGL(compress_gated_slice_kernel<DT_F32>, grid, dim3(cmp::kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL(compress_gated_slice_kernel<DT_BF16>, grid, dim3(cmp::kThreads), 0, stream, a);
        return hipGetLastError();
    }
    if (a.tok_dtype == DT_F32)
        hipLaunchKernelGGL(compress_gated_kernel<DT_F32>, dim3(total_new), dim3(kGatedThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(compress_gated_kernel<DT_BF16>, dim3(total_new), dim3(kGatedThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lcca
