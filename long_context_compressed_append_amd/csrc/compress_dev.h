// Device code of compress_append, shared by its own kernel and by the decode
// launch that runs it beside the top-k selection.
// compress_append: fold each completed group of m tokens into one entry by a
// softmax-weighted sum (one scalar logit per token), encode it into the paged
// pool, write new tokens into the window ring and the remainder ring.
//
// [Page "vLLM uveo DeepSeek V4 s 8,7x manjim KV cacheom", section "Kako
//  funkcionira optimizacija KV cachea?": tokens are aggregated by weighted
//  summation (4x to 128x); section "Sto je vLLM morao rijesiti u
//  integraciji?": 256-position logical blocks per layer, remainder of the
//  compressor kept as sliding-window state.]
//
// Grid: (new token t, slice s).  Slices 0 .. SK-1 cover 64-dimension blocks
// of the shared-KV stream, SK .. SK+SI-1 those of the indexer-key stream,
// slice SK+SI the token's ring writes.
//   * A token that completes group g makes each of its compression slices
//     aggregate the slice's 64 dimensions of the group: 256 threads = 32
//     token lanes x 8 dimension chunks of 8.  The group's token bytes, its
//     logits and the pool row's block-table entry are all requested first,
//     so they travel together; the softmax weights, the weighted sum (token
//     lanes reduced in LDS), the encode (bf16 / MXFP4 / FP8 / fp32) and the
//     store into the pool follow.
//   * The ring slice writes the token into the window ring if it is among
//     the last `capacity` tokens of its chunk (FP8 with a per-token scale)
//     and, if it belongs to the chunk's incomplete tail, into the remainder
//     ring.  One case needs ordering: a chunk that starts inside a group,
//     completes that group and ends inside a later group reads ring slots it
//     also rewrites.  Then slice 0 of the token completing the first group
//     aggregates that whole group (all slices, both streams) and writes the
//     tail after its reads.
#pragma once
#include "device.h"
#include "kernels.h"

namespace lcca {
namespace {
namespace cmp {

constexpr int kThreads = 256;
constexpr int kSliceDims = 64;               // dimensions per slice
constexpr int kChunk = 8;                    // dimensions per thread
constexpr int kLanes = kThreads / (kSliceDims / kChunk);   // token lanes = 32
constexpr int kMaxPairsPerThread = 4;        // window encode: dim <= 2048

template <int TOK>
__device__ inline void load_pair(const void* base, int64_t elem, float& x0, float& x1) {
    if (TOK == DT_F32) {
        float2 v = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(base) + elem);
        x0 = v.x; x1 = v.y;
    } else {
        uint32_t v = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(base) + elem);
        x0 = bf16_to_f32(v & 0xffffu); x1 = bf16_to_f32(v >> 16);
    }
}

// Block-wide max of non-negative values (all threads get the result).
__device__ inline float block_max(float v, float* red) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
    return r;
}

// Store one (even, odd) channel pair of row `row` in window dtype `dt`
// (F32 or BF16).
__device__ inline void store_pair(int dt, uint8_t* data, int64_t row, int dim, int pair, float x0, float x1) {
    if (dt == DT_F32) *reinterpret_cast<float2*>(data + row * 4LL * dim + 8LL * pair) = make_float2(x0, x1);
    else *reinterpret_cast<uint32_t*>(data + row * 2LL * dim + 4LL * pair) = pack_bf16x2(x0, x1);
}

struct SeqChunk {
    int b, start, end, n;
    int64_t c0;
};

constexpr int kSeqLds = 1024;                 // batches up to this size search in LDS

// Sequence of token t: the largest b with cu_new[b] <= t.  For batches of up
// to kSeqLds sequences, cu_new and start_pos are first copied to LDS in one
// round of loads (by the NT threads of the workgroup), so the search costs no
// dependent global loads.
template <int NT = kThreads>
__device__ inline SeqChunk seq_of(const CompressArgs& p, int t, int* cu_lds, int* sp_lds) {
    const bool in_lds = p.batch <= kSeqLds;
    if (in_lds) {
        for (int i = threadIdx.x; i <= p.batch; i += NT) {
            cu_lds[i] = p.cu_new[i];
            if (i < p.batch) sp_lds[i] = p.start_pos[i];
        }
        __syncthreads();
    }
    auto cu = [&](int i) { return in_lds ? cu_lds[i] : p.cu_new[i]; };
    int lo = 0, hi = p.batch - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu(mid) <= t) lo = mid; else hi = mid - 1;
    }
    SeqChunk q;
    q.b = lo;
    q.c0 = cu(lo);
    q.n = cu(lo + 1) - (int)q.c0;
    q.start = in_lds ? sp_lds[lo] : p.start_pos[lo];
    if (chunk_invalid(t, (int)q.c0, (int)q.c0 + q.n, q.start, p.total_new, p.max_blocks, p.dbg, kDbgChunk)) {
        q.c0 = t; q.n = 1; q.start = 0;           // (debug builds) a chunk of this token alone at position 0
    }
    q.end = q.start + q.n;
    return q;
}

constexpr int kMaxTokPerLane = 256 / kLanes;   // m <= 256

// Raw bytes of one token's 8-dimension chunk: one 16-byte load for bf16,
// two for fp32.
template <int TOK>
struct RawChunk {
    u32x4 v[TOK == DT_F32 ? 2 : 1];
};

template <int TOK>
__device__ __forceinline__ void load_chunk(const void* base, int64_t elem, RawChunk<TOK>& r) {
    if constexpr (TOK == DT_F32) {
        const u32x4* q = reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(base) + elem);
        r.v[0] = q[0];
        r.v[1] = q[1];
    } else {
        r.v[0] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + elem);
    }
}

template <int TOK>
__device__ __forceinline__ void unpack_chunk(const RawChunk<TOK>& r, float (&x)[kChunk]) {
    if constexpr (TOK == DT_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[i] = __uint_as_float(r.v[0][i]); x[4 + i] = __uint_as_float(r.v[1][i]); }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_to_f32(r.v[0][i] & 0xffffu);
            x[2 * i + 1] = bf16_to_f32(r.v[0][i] >> 16);
        }
    }
}

// Everything one slice of group g reads from memory, requested up front.
template <int TOK>
struct SliceLoads {
    RawChunk<TOK> tok[kMaxTokPerLane];   // token lane's chunks, tokens lane + 32 j
    float logit;                         // logit of token `tid` of the group (threads < m)
    int64_t row;                         // pool row of the entry
};

template <int TOK>
__device__ __forceinline__ void issue_slice(const CompressArgs& p, const SeqChunk& q, int g, bool ik_stream, int d0,
                                            SliceLoads<TOK>& L) {
    const int m = p.m;
    const int dim = ik_stream ? p.dI : p.D;
    const void* tok = ik_stream ? p.ik_tok : p.kv_tok;
    const void* rtok = ik_stream ? p.rem_ik : p.rem_kv;
    const float* lg = ik_stream ? p.ik_logit : p.kv_logit;
    const float* rlg = ik_stream ? p.rem_ik_logit : p.rem_kv_logit;
    const int tid = threadIdx.x;
    const int lane = tid / (kSliceDims / kChunk), ch = tid % (kSliceDims / kChunk);
    const int d = d0 + ch * kChunk;
    const bool active = d < dim;
#pragma unroll
    for (int j = 0; j < kMaxTokPerLane; ++j) {
        const int i = lane + kLanes * j;
        if (active && i < m) {
            const int t = g * m + i;
            if (t >= q.start) load_chunk<TOK>(tok, (q.c0 + (t - q.start)) * dim + d, L.tok[j]);
            else load_chunk<TOK>(rtok, ((int64_t)q.b * m + t % m) * dim + d, L.tok[j]);
        }
    }
    L.logit = -INFINITY;
    if (tid < m) {
        const int t = g * m + tid;
        L.logit = t >= q.start ? lg[q.c0 + (t - q.start)] : rlg[(int64_t)q.b * m + t % m];
    }
    const int E = 256 / m;
    L.row = (int64_t)checked(p.block_table[(int64_t)q.b * p.max_blocks + g / E], 0, p.n_blocks - 1, p.dbg, kDbgBlock) * E +
            g % E;
}

// Softmax weights of the group's logits (thread i < m holds logit i) into
// w_lds (m <= 256).  Groups of up to 64 tokens are done by wave 0 alone.
__device__ void group_weights(int m, float a, float* w_lds, float* red) {
    const int tid = threadIdx.x;
    if (m <= 64) {
        if (tid < 64) {
            const float mx = wave_max(a);
            const float e = tid < m ? expf(a - mx) : 0.0f;
            const float s = wave_sum(e);
            if (tid < m) w_lds[tid] = e / s;
        }
        __syncthreads();
        return;
    }
    float mx = wave_max(a);
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float e = tid < m ? expf(a - mx) : 0.0f;
    float s = wave_sum(e);
    __syncthreads();
    if ((tid & 63) == 0) red[4 + (tid >> 6)] = s;
    __syncthreads();
    s = red[4] + red[5] + red[6] + red[7];
    if (tid < m) w_lds[tid] = e / s;
    __syncthreads();
}

// Encode dimension dim_i of an entry (value v) into pool row `row` of a
// stream; called by the 64 threads of wave 0, thread i holding dimension
// d0 + i of a 64-dimension slice (MXFP4 blocks of 32 dimensions are its two
// half-waves; dimensions beyond the stream's take part in the exchanges
// only).
__device__ __forceinline__ void store_slice_dim(const CompressArgs& p, bool ik_stream, int64_t row, int dim_i,
                                                float v) {
    const int dim = ik_stream ? p.dI : p.D;
    const int dt = ik_stream ? p.ik_dtype : p.kv_dtype;
    uint8_t* data = reinterpret_cast<uint8_t*>(ik_stream ? p.ik_data : p.kv_data);
    const bool in = dim_i < dim;
    if (dt == DT_MXFP4) {
        float a = in ? fabsf(v) : 0.0f;
        a = fmaxf(a, lane_xor<16>(a));
        a = fmaxf(a, lane_xor<8>(a));
        a = fmaxf(a, lane_xor<4>(a));
        a = fmaxf(a, lane_xor<2>(a));
        a = fmaxf(a, lane_xor<1>(a));
        const int X = mx_scale_exp(a);
        const uint32_t c = fp4_code(ldexpf(v, -X));
        // lane i + 1's code (row_shl:1; used by even lanes, whose partner is in their row)
        const uint32_t c_hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)c, 0x101, 0xF, 0xF, false);
        if (in && (dim_i & 1) == 0) data[row * (int64_t)(dim / 2) + dim_i / 2] = (uint8_t)(c | (c_hi << 4));
        if (in && (dim_i & 31) == 0)
            reinterpret_cast<uint8_t*>(p.kv_scale)[row * (int64_t)(dim / 32) + dim_i / 32] = (uint8_t)(X + 127);
    } else if (in) {
        if (dt == DT_F32) reinterpret_cast<float*>(data)[row * dim + dim_i] = v;
        else if (dt == DT_BF16) reinterpret_cast<uint16_t*>(data)[row * dim + dim_i] = (uint16_t)f32_to_bf16(v);
        else data[row * (int64_t)dim + dim_i] = (uint8_t)f32_to_fp8(v);
    }
}

// Weighted sum of dimensions [d0, d0 + 64) of the group over its tokens
// (loaded by issue_slice, weights in w_lds), encoded into the pool.
template <int TOK>
__device__ void reduce_slice(const CompressArgs& p, bool ik_stream, int d0, const SliceLoads<TOK>& L,
                             const float* w_lds, float* red) {
    const int m = p.m;
    const int dim = ik_stream ? p.dI : p.D;
    const int tid = threadIdx.x;
    const int lane = tid / (kSliceDims / kChunk), ch = tid % (kSliceDims / kChunk);
    const int d = d0 + ch * kChunk;
    const bool active = d < dim;

    float acc[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxTokPerLane; ++j) {
        const int i = lane + kLanes * j;
        if (active && i < m) {
            float x[kChunk];
            unpack_chunk<TOK>(L.tok[j], x);
            const float w = w_lds[i];
#pragma unroll
            for (int e = 0; e < kChunk; ++e) acc[e] = fmaf(w, x[e], acc[e]);
        }
    }
    // reduce over the token lanes: red[lane][64]
#pragma unroll
    for (int e = 0; e < kChunk; ++e) red[lane * kSliceDims + ch * kChunk + e] = acc[e];
    __syncthreads();
    float v = 0.0f;
    const int dd = tid;                                        // dimension d0 + dd, threads < 64
    if (tid < kSliceDims) {
        const int nl = min(m, kLanes);                         // token lanes holding tokens
        for (int l = 0; l < nl; ++l) v += red[l * kSliceDims + dd];
    }
    if (tid < kSliceDims) store_slice_dim(p, ik_stream, L.row, d0 + dd, v);
    __syncthreads();                                           // red is reused by the next slice
}

// One slice of group g, start to finish.
template <int TOK>
__device__ void compress_slice(const CompressArgs& p, const SeqChunk& q, int g, bool ik_stream, int d0, float* w_lds,
                               float* red) {
    SliceLoads<TOK> L;
    issue_slice<TOK>(p, q, g, ik_stream, d0, L);
    group_weights(p.m, L.logit, w_lds, red);
    reduce_slice<TOK>(p, ik_stream, d0, L, w_lds, red);
}

template <int TOK>
__device__ __forceinline__ void write_ring(const CompressArgs& p, const SeqChunk& q, int tt) {
    const int m = p.m;
    const int esz = TOK == DT_F32 ? 4 : 2;
    const int64_t src = q.c0 + (tt - q.start);
    const int64_t slot = (int64_t)q.b * m + tt % m;
    const uint8_t* s8 = reinterpret_cast<const uint8_t*>(p.kv_tok) + src * p.D * esz;
    uint8_t* d8 = reinterpret_cast<uint8_t*>(p.rem_kv) + slot * p.D * esz;
    for (int i = threadIdx.x; i < p.D * esz / 4; i += kThreads)
        reinterpret_cast<uint32_t*>(d8)[i] = reinterpret_cast<const uint32_t*>(s8)[i];
    if (threadIdx.x == 0) p.rem_kv_logit[slot] = p.kv_logit[src];
    if (p.ik_data != nullptr) {
        const uint8_t* si = reinterpret_cast<const uint8_t*>(p.ik_tok) + src * p.dI * esz;
        uint8_t* di = reinterpret_cast<uint8_t*>(p.rem_ik) + slot * p.dI * esz;
        for (int i = threadIdx.x; i < p.dI * esz / 4; i += kThreads)
            reinterpret_cast<uint32_t*>(di)[i] = reinterpret_cast<const uint32_t*>(si)[i];
        if (threadIdx.x == 0) p.rem_ik_logit[slot] = p.ik_logit[src];
    }
}

// New token t (position pos of its chunk) into its window slot if it is
// among the chunk's last `capacity` tokens (FP8: a per-token scale from the
// block-wide max; `red` holds at least 8 floats of LDS).
template <int TOK>
__device__ void write_window(const CompressArgs& p, const SeqChunk& q, int t, int pos, float* red) {
    const int tid = threadIdx.x, D = p.D;
    if (p.win_data != nullptr && pos >= q.end - p.win_cap) {
        const int64_t slot = (int64_t)q.b * p.win_cap + pos % p.win_cap;
        uint8_t* wd = reinterpret_cast<uint8_t*>(p.win_data);
        const int pairs = D / 2;
        if (p.win_dtype == DT_FP8) {
            float x0[kMaxPairsPerThread], x1[kMaxPairsPerThread];
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < kMaxPairsPerThread; ++i) {
                const int pr = tid + i * kThreads;
                x0[i] = x1[i] = 0.0f;
                if (pr < pairs) load_pair<TOK>(p.kv_tok, (int64_t)t * D + 2 * pr, x0[i], x1[i]);
                amax = fmaxf(amax, fmaxf(fabsf(x0[i]), fabsf(x1[i])));
            }
            amax = block_max(amax, red);
            const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
            if (tid == 0) p.win_scale[slot] = sc;
#pragma unroll
            for (int i = 0; i < kMaxPairsPerThread; ++i) {
                const int pr = tid + i * kThreads;
                if (pr < pairs) {
                    const uint32_t c = f32_to_fp8(x0[i] / sc) | (f32_to_fp8(x1[i] / sc) << 8);
                    *reinterpret_cast<uint16_t*>(wd + slot * D + 2 * pr) = (uint16_t)c;
                }
            }
        } else {
            for (int pr = tid; pr < pairs; pr += kThreads) {
                float x0, x1;
                load_pair<TOK>(p.kv_tok, (int64_t)t * D + 2 * pr, x0, x1);
                store_pair(p.win_dtype, wd, slot, D, pr, x0, x1);
            }
        }
    }
}


// The whole work of grid item (new token t, slice s) on threads 0 .. 255 of
// a workgroup (a larger workgroup's other waves must have exited).
template <int TOK>
__device__ __forceinline__ void compress_append_body(const CompressArgs& p, int t, int s) {
    __shared__ float w_lds[256];
    __shared__ float red[kLanes * kSliceDims];
    __shared__ int cu_lds[kSeqLds + 1], sp_lds[kSeqLds];
    const SeqChunk q = seq_of(p, t, cu_lds, sp_lds);
    const int pos = q.start + (t - (int)q.c0);
    const int m = p.m, D = p.D;
    const int SK = (D + kSliceDims - 1) / kSliceDims;
    const int SI = p.ik_data != nullptr ? (p.dI + kSliceDims - 1) / kSliceDims : 0;
    const int g0 = q.start / m;                                // group holding `start`
    const bool race = (q.start % m) != 0 && (q.end % m) != 0 && q.end >= (g0 + 1) * m;
    const int tail0 = max((q.end / m) * m, q.start);

    if (s == SK + SI) {
        // (1) window ring
        write_window<TOK>(p, q, t, pos, red);
        // (3) remainder ring: each tail token writes itself (see the header
        // comment for `race`)
        if (!race && pos >= tail0) write_ring<TOK>(p, q, pos);
        return;
    }

    // (2) the group this token completes
    if ((pos + 1) % m == 0) {
        const int g = pos / m;
        if (race && g == g0) {
            // whole first group here, then the tail of the chunk into the ring
            if (s == 0) {
                for (int k = 0; k < SK; ++k) compress_slice<TOK>(p, q, g, false, k * kSliceDims, w_lds, red);
                for (int k = 0; k < SI; ++k) compress_slice<TOK>(p, q, g, true, k * kSliceDims, w_lds, red);
                __syncthreads();
                for (int tt = tail0; tt < q.end; ++tt) write_ring<TOK>(p, q, tt);
            }
        } else {
            const bool ik = s >= SK;
            compress_slice<TOK>(p, q, g, ik, (ik ? s - SK : s) * kSliceDims, w_lds, red);
        }
    }
}

}  // namespace cmp
}  // namespace
}  // namespace lcca
