// compress_append: fold each completed group of m tokens into one entry by a
// softmax-weighted sum (one scalar logit per token), encode it into the paged
// pool, write new tokens into the window ring and the remainder ring.
//
// [P1 = page "vLLM uveo DeepSeek V4 s 8,7x manjim KV cacheom", section
//  "Kako funkcionira optimizacija KV cachea?": tokens are aggregated by
//  weighted summation (4x to 128x); section "Sto je vLLM morao rijesiti u
//  integraciji?": 256-position logical blocks per layer, remainder of the
//  compressor kept as sliding-window state.]
//
// One workgroup per new token (HBM/latency bound, no reuse to exploit):
//   * if the token is among the last `capacity` of its sequence's chunk, it is
//     encoded into the window ring;
//   * if it completes a group (pos+1 multiple of m), the block aggregates the
//     group (tokens older than the chunk come from the remainder ring) for the
//     KV stream and the indexer-key stream and stores both entries;
//   * exactly one block per sequence writes the chunk's incomplete tail into
//     the remainder ring: the block that read the ring (if any), after its
//     reads, so no other block can observe a half-updated ring.
#include "device.h"
#include "kernels.h"

namespace lcca {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxPairsPerThread = 4;        // dim <= 2048

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

// Store one (even, odd) channel pair of row `row` in pool/ring dtype `dt`.
// MXFP4 needs the 16 threads of a 32-channel block to be active together;
// `amax32` is their shared block maximum.
__device__ inline void store_pair(int dt, uint8_t* data, uint8_t* scale_mx, int64_t row, int dim, int pair,
                                  float x0, float x1) {
    switch (dt) {
    case DT_F32:
        *reinterpret_cast<float2*>(data + row * 4LL * dim + 8LL * pair) = make_float2(x0, x1);
        break;
    case DT_BF16:
        *reinterpret_cast<uint32_t*>(data + row * 2LL * dim + 4LL * pair) = pack_bf16x2(x0, x1);
        break;
    case DT_FP8:
        *reinterpret_cast<uint16_t*>(data + row * (int64_t)dim + 2LL * pair) =
            (uint16_t)(f32_to_fp8(x0) | (f32_to_fp8(x1) << 8));
        break;
    case DT_MXFP4: {
        float a = fmaxf(fabsf(x0), fabsf(x1));
        for (int o = 8; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));   // 16 lanes = 32 channels
        int X = mx_scale_exp(a);
        uint32_t c0 = fp4_code(ldexpf(x0, -X)), c1 = fp4_code(ldexpf(x1, -X));
        data[row * (int64_t)(dim / 2) + pair] = (uint8_t)(c0 | (c1 << 4));
        if ((pair & 15) == 0) scale_mx[row * (int64_t)(dim / 32) + pair / 16] = (uint8_t)(X + 127);
        break;
    }
    }
}

template <int TOK>
__device__ void compress_group(const CompressArgs& p, int b, int64_t c0, int start, int g, bool ik_stream,
                               float* w_lds) {
    const int m = p.m;
    const int dim = ik_stream ? p.dI : p.D;
    const void* tok = ik_stream ? p.ik_tok : p.kv_tok;
    const float* lg = ik_stream ? p.ik_logit : p.kv_logit;
    const void* rtok = ik_stream ? p.rem_ik : p.rem_kv;
    const float* rlg = ik_stream ? p.rem_ik_logit : p.rem_kv_logit;
    const int tid = threadIdx.x;

    // softmax weights of the group's m logits (m <= 256)
    __syncthreads();
    if (tid < m) {
        int t = g * m + tid;
        w_lds[tid] = t >= start ? lg[c0 + (t - start)] : rlg[(int64_t)b * m + t % m];
    }
    __syncthreads();
    if (tid < 64) {
        float mx = -INFINITY;
        for (int i = tid; i < m; i += 64) mx = fmaxf(mx, w_lds[i]);
        mx = wave_max(mx);
        float s = 0.0f;
        for (int i = tid; i < m; i += 64) s += expf(w_lds[i] - mx);
        s = wave_sum(s);
        for (int i = tid; i < m; i += 64) w_lds[i] = expf(w_lds[i] - mx) / s;
    }
    __syncthreads();

    const int pairs = dim / 2;
    const int E = 256 / m;
    const int64_t blk = p.block_table[(int64_t)b * p.max_blocks + g / E];
    const int64_t row = blk * E + g % E;
    const int dt = ik_stream ? p.ik_dtype : p.kv_dtype;
    uint8_t* data = reinterpret_cast<uint8_t*>(ik_stream ? p.ik_data : p.kv_data);
    uint8_t* scale = reinterpret_cast<uint8_t*>(ik_stream ? p.ik_scale : p.kv_scale);
    for (int pr = tid; pr < pairs; pr += kThreads) {
        float a0 = 0.0f, a1 = 0.0f;
        for (int i = 0; i < m; ++i) {
            int t = g * m + i;
            float x0, x1;
            if (t >= start) load_pair<TOK>(tok, (c0 + (t - start)) * dim + 2 * pr, x0, x1);
            else load_pair<TOK>(rtok, ((int64_t)b * m + t % m) * dim + 2 * pr, x0, x1);
            const float w = w_lds[i];
            a0 = fmaf(w, x0, a0);
            a1 = fmaf(w, x1, a1);
        }
        store_pair(dt, data, scale, row, dim, pr, a0, a1);
    }
}

template <int TOK>
__global__ __launch_bounds__(kThreads) void compress_append_kernel(CompressArgs p) {
    __shared__ float w_lds[256];
    __shared__ float red[kThreads / 64];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    // sequence of this token: the largest b with cu_new[b] <= t
    int lo = 0, hi = p.batch - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (p.cu_new[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int64_t c0 = p.cu_new[b];
    const int n = p.cu_new[b + 1] - (int)c0;
    const int start = p.start_pos[b];
    const int end = start + n;
    const int pos = start + (t - (int)c0);
    const int m = p.m;
    const int D = p.D;

    // (1) window ring
    if (p.win_data != nullptr && pos >= end - p.win_cap) {
        const int64_t slot = (int64_t)b * p.win_cap + pos % p.win_cap;
        uint8_t* wd = reinterpret_cast<uint8_t*>(p.win_data);
        const int pairs = D / 2;
        if (p.win_dtype == DT_FP8) {
            float x0[kMaxPairsPerThread], x1[kMaxPairsPerThread];
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < kMaxPairsPerThread; ++i) {
                int pr = tid + i * kThreads;
                x0[i] = x1[i] = 0.0f;
                if (pr < pairs) load_pair<TOK>(p.kv_tok, (int64_t)t * D + 2 * pr, x0[i], x1[i]);
                amax = fmaxf(amax, fmaxf(fabsf(x0[i]), fabsf(x1[i])));
            }
            amax = block_max(amax, red);
            const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
            if (tid == 0) p.win_scale[slot] = s;
#pragma unroll
            for (int i = 0; i < kMaxPairsPerThread; ++i) {
                int pr = tid + i * kThreads;
                if (pr < pairs) {
                    uint32_t c = f32_to_fp8(x0[i] / s) | (f32_to_fp8(x1[i] / s) << 8);
                    *reinterpret_cast<uint16_t*>(wd + slot * D + 2 * pr) = (uint16_t)c;
                }
            }
        } else {
            for (int pr = tid; pr < pairs; pr += kThreads) {
                float x0, x1;
                load_pair<TOK>(p.kv_tok, (int64_t)t * D + 2 * pr, x0, x1);
                store_pair(p.win_dtype, wd, nullptr, slot, D, pr, x0, x1);
            }
        }
    }

    // (2) group completed by this token
    if ((pos + 1) % m == 0) {
        const int g = pos / m;
        compress_group<TOK>(p, b, c0, start, g, false, w_lds);
        if (p.ik_data != nullptr) compress_group<TOK>(p, b, c0, start, g, true, w_lds);
    }

    // (3) remainder ring: the incomplete tail of the chunk
    const int g0_end = (start / m + 1) * m;                    // end of the group holding `start`
    const int writer = (start % m != 0 && end >= g0_end) ? g0_end - 1 : start;
    if (pos == writer) {
        __syncthreads();                                       // ring reads of step (2) are done
        int tail0 = (end / m) * m;
        if (tail0 < start) tail0 = start;
        const int esz = TOK == DT_F32 ? 4 : 2;
        for (int tt = tail0; tt < end; ++tt) {
            const int64_t src = c0 + (tt - start);
            const int64_t slot = (int64_t)b * m + tt % m;
            const uint8_t* s8 = reinterpret_cast<const uint8_t*>(p.kv_tok) + src * D * esz;
            uint8_t* d8 = reinterpret_cast<uint8_t*>(p.rem_kv) + slot * D * esz;
            for (int i = tid; i < D * esz / 4; i += kThreads)
                reinterpret_cast<uint32_t*>(d8)[i] = reinterpret_cast<const uint32_t*>(s8)[i];
            if (tid == 0) p.rem_kv_logit[slot] = p.kv_logit[src];
            if (p.ik_data != nullptr) {
                const uint8_t* si = reinterpret_cast<const uint8_t*>(p.ik_tok) + src * p.dI * esz;
                uint8_t* di = reinterpret_cast<uint8_t*>(p.rem_ik) + slot * p.dI * esz;
                for (int i = tid; i < p.dI * esz / 4; i += kThreads)
                    reinterpret_cast<uint32_t*>(di)[i] = reinterpret_cast<const uint32_t*>(si)[i];
                if (tid == 0) p.rem_ik_logit[slot] = p.ik_logit[src];
            }
        }
    }
}

}  // namespace

hipError_t launch_compress_append(const CompressArgs& a, int total_new, hipStream_t stream) {
    if (total_new <= 0) return hipSuccess;
    if (a.tok_dtype == DT_F32)
        hipLaunchKernelGGL(compress_append_kernel<DT_F32>, dim3(total_new), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(compress_append_kernel<DT_BF16>, dim3(total_new), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lcca
