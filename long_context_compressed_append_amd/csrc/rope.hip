// Rotary position embedding of a slice of dimensions, in place, and its
// inverse.
//
// The shared key/value vectors carry RoPE dimensions and the attention
// output is rotated back by the inverse rotation [P1 "Kako funkcionira
// optimizacija KV cachea?"].  The pages fix no convention; the caller gives
// it: the slice [off, off + rd) of each head vector, the pairing (pair i is
// dims (2i, 2i+1) or (i, i + rd/2)) and the pair frequencies (fp32, computed
// by the host from a base or passed in).  Pair i of row r is rotated by the
// fp32 angle fp32(pos[r]) * freq[i] (by its negative for the inverse).
//
// HBM-bound elementwise work (read and write of the slice): each thread owns
// G consecutive pairs of one row, forms their cos/sin once, and applies them
// to a run of the row's heads, loading a batch of heads before storing any so
// that loads overlap.  Consecutive lanes take consecutive pairs, so a wave
// reads and writes contiguous runs of each head's slice.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device.h"
#include "kernels.h"

namespace lcca {
namespace {

constexpr int kRopeThreads = 256;
constexpr int kRopeHeadBatch = 4;

// N contiguous elements of x (f32 or bf16) <-> N floats.  The host
// guarantees the alignment of the widest access (16 bytes).
template <bool BF16, int N>
__device__ __forceinline__ void load_run(const void* p, float* v) {
    if constexpr (BF16) {
        const uint16_t* q = (const uint16_t*)p;
        if constexpr (N == 8) {
            const uint4 w = *(const uint4*)q;
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_to_f32(u[i] & 0xffffu); v[2 * i + 1] = bf16_to_f32(u[i] >> 16); }
        } else if constexpr (N == 4) {
            const uint2 w = *(const uint2*)q;
            v[0] = bf16_to_f32(w.x & 0xffffu); v[1] = bf16_to_f32(w.x >> 16);
            v[2] = bf16_to_f32(w.y & 0xffffu); v[3] = bf16_to_f32(w.y >> 16);
        } else {
#pragma unroll
            for (int i = 0; i < N; ++i) v[i] = bf16_to_f32(q[i]);
        }
    } else {
        const float* q = (const float*)p;
        if constexpr (N % 4 == 0) {
#pragma unroll
            for (int i = 0; i < N; i += 4) {
                const float4 w = *(const float4*)(q + i);
                v[i] = w.x; v[i + 1] = w.y; v[i + 2] = w.z; v[i + 3] = w.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < N; ++i) v[i] = q[i];
        }
    }
}

template <bool BF16, int N>
__device__ __forceinline__ void store_run(void* p, const float* v) {
    if constexpr (BF16) {
        uint16_t* q = (uint16_t*)p;
        if constexpr (N == 8) {
            *(uint4*)q = uint4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                               pack_bf16x2(v[6], v[7])};
        } else if constexpr (N == 4) {
            *(uint2*)q = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        } else {
#pragma unroll
            for (int i = 0; i < N; ++i) q[i] = (uint16_t)f32_to_bf16(v[i]);
        }
    } else {
        float* q = (float*)p;
        if constexpr (N % 4 == 0) {
#pragma unroll
            for (int i = 0; i < N; i += 4) *(float4*)(q + i) = float4{v[i], v[i + 1], v[i + 2], v[i + 3]};
        } else {
#pragma unroll
            for (int i = 0; i < N; ++i) q[i] = v[i];
        }
    }
}

// The G pairs a thread owns, for one head: a = first members, b = second.
// Interleaved: 2G contiguous elements (a0 b0 a1 b1 ...); half split: G
// contiguous first members and the G second members rd/2 further on.
template <bool BF16, bool HALF, int G>
__device__ __forceinline__ void load_pairs(const char* base, int half, int esz, float* a, float* b) {
    if constexpr (HALF) {
        load_run<BF16, G>(base, a);
        load_run<BF16, G>(base + (int64_t)half * esz, b);
    } else {
        float v[2 * G];
        load_run<BF16, 2 * G>(base, v);
#pragma unroll
        for (int j = 0; j < G; ++j) { a[j] = v[2 * j]; b[j] = v[2 * j + 1]; }
    }
}

template <bool BF16, bool HALF, int G>
__device__ __forceinline__ void store_pairs(char* base, int half, int esz, const float* a, const float* b) {
    if constexpr (HALF) {
        store_run<BF16, G>(base, a);
        store_run<BF16, G>(base + (int64_t)half * esz, b);
    } else {
        float v[2 * G];
#pragma unroll
        for (int j = 0; j < G; ++j) { v[2 * j] = a[j]; v[2 * j + 1] = b[j]; }
        store_run<BF16, 2 * G>(base, v);
    }
}

template <bool BF16, bool HALF, int G>
__global__ __launch_bounds__(kRopeThreads) void rope_kernel(RopeArgs a) {
    constexpr int esz = BF16 ? 2 : 4;
    const int npg = a.rd / 2 / G;                  // pair groups per head
    const int64_t total = a.rows * (int64_t)a.nchunks * npg;
    const int half = a.rd / 2;
    for (int64_t t = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * kRopeThreads) {
        const int pg = (int)(t % npg);
        const int64_t rc = t / npg;
        const int chunk = (int)(rc % a.nchunks);
        const int64_t row = rc / a.nchunks;
        const float p = (float)a.pos[row];
        float c[G], s[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            sincosf(p * a.freq[pg * G + j], &s[j], &c[j]);
            if (a.inverse) s[j] = -s[j];
        }
        const int h0 = chunk * a.hchunk;
        const int h1 = min(a.heads, h0 + a.hchunk);
        // offset of the thread's first element in head h0 of the row
        const int first = a.off + (HALF ? pg * G : 2 * pg * G);
        char* base = (char*)a.x + ((row * a.heads + h0) * (int64_t)a.dim + first) * esz;
        const int64_t hstride = (int64_t)a.dim * esz;
        for (int h = h0; h < h1; h += kRopeHeadBatch) {
            const int nb = min(kRopeHeadBatch, h1 - h);
            float va[kRopeHeadBatch][G], vb[kRopeHeadBatch][G];
#pragma unroll
            for (int u = 0; u < kRopeHeadBatch; ++u)
                if (u < nb) load_pairs<BF16, HALF, G>(base + u * hstride, half, esz, va[u], vb[u]);
#pragma unroll
            for (int u = 0; u < kRopeHeadBatch; ++u) {
                if (u < nb) {
                    float ra[G], rb[G];
#pragma unroll
                    for (int j = 0; j < G; ++j) {
                        ra[j] = va[u][j] * c[j] - vb[u][j] * s[j];
                        rb[j] = va[u][j] * s[j] + vb[u][j] * c[j];
                    }
                    store_pairs<BF16, HALF, G>(base + u * hstride, half, esz, ra, rb);
                }
            }
            base += kRopeHeadBatch * hstride;
        }
    }
}

template <bool BF16, bool HALF>
hipError_t launch_g(const RopeArgs& a, int G, int blocks, hipStream_t st) {
    if (G == 4)
        rope_kernel<BF16, HALF, 4><<<blocks, kRopeThreads, 0, st>>>(a);
    else
        rope_kernel<BF16, HALF, 1><<<blocks, kRopeThreads, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace

int rope_pairs_per_thread(const RopeArgs& a) {
    const bool aligned = ((uintptr_t)a.x % 16 == 0) && a.off % 8 == 0 && a.rd % 8 == 0 && a.dim % 8 == 0;
    return aligned ? 4 : 1;
}

hipError_t launch_rope(RopeArgs a, hipStream_t st) {
    const int G = rope_pairs_per_thread(a);
    const int64_t npg = a.rd / 2 / G;
    // split a row's heads over threads until there are about 2^17 threads
    const int64_t per_row = npg;
    int64_t nchunks = (131072 + a.rows * per_row - 1) / (a.rows * per_row);
    nchunks = std::max<int64_t>(1, std::min<int64_t>(nchunks, a.heads));
    a.hchunk = (int)((a.heads + nchunks - 1) / nchunks);
    a.nchunks = (a.heads + a.hchunk - 1) / a.hchunk;
    const int64_t total = a.rows * a.nchunks * npg;
    const int blocks = (int)std::min<int64_t>((total + kRopeThreads - 1) / kRopeThreads, 1 << 16);
    if (a.bf16)
        return a.half_split ? launch_g<true, true>(a, G, blocks, st) : launch_g<true, false>(a, G, blocks, st);
    return a.half_split ? launch_g<false, true>(a, G, blocks, st) : launch_g<false, false>(a, G, blocks, st);
}

}  // namespace lcca
