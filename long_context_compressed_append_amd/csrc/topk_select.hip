// topk_select: for each query row, the k visible entries with the largest
// indexer logits (equal logits: smaller entry first), written in ascending
// entry order and padded with -1.  [Page "vLLM uveo DeepSeek V4 s 8,7x manjim
// KV cacheom", section "Kako funkcionira optimizacija KV cachea?": attention is
// limited to the top-k compressed tokens.]
//
// One 1024-thread workgroup per row; thread i owns the contiguous entries
// [i*C, (i+1)*C).  Logits map to order-preserving u32 keys (-0.0 folded onto
// +0.0).  Rows of up to 32K entries are held in registers; longer rows are
// re-read from memory on every pass.
//   1. A block min/max of the keys gives their common leading bits, so the
//      radix digits start at the first bit in which the keys differ.
//   2. Radix passes of up to 8 bits find the k-th largest key T and how many
//      keys equal to T are still needed.  Histograms live in LDS as 16 copies
//      selected by lane, so lanes holding the same digit rarely hit the same
//      counter.
//   3. A final pass in entry order keeps every key > T and the first `need`
//      keys == T; block-wide exclusive scans give each kept entry its output
//      slot, so the result is deterministic and sorted by entry.
#include "device.h"
#include "kernels.h"

namespace lcca {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kCopies = 16;

__device__ inline uint32_t order_key(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;                               // -0.0 ties +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan over the block (thread order); returns this thread's prefix
// and writes the block total to *total.
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t inc = v;
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t t = __shfl_up(inc, o);
        if (lane >= o) inc += t;
    }
    __syncthreads();
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    uint32_t before = 0, tot = 0;
    for (int i = 0; i < kWaves; ++i) {
        uint32_t s = wsum[i];
        if (i < w) before += s;
        tot += s;
    }
    *total = tot;
    return before + inc - v;
}

// Keys of this thread's chunk: resident in registers (R > 0) or streamed.
template <int R>
struct Chunk {
    uint32_t u[R > 0 ? R : 1];
    int c0, c1;                 // entry range [c0, c1)
    const float* L;

    // per_thread is a multiple of 4; with `vec` the row is 16-byte aligned and
    // the chunk is read with 16-byte loads.
    __device__ void init(const float* logits, int n, int per_thread, bool vec) {
        L = logits;
        c0 = min((int)threadIdx.x * per_thread, n);
        c1 = min(c0 + per_thread, n);
        if (R > 0) {
            if (vec) {
#pragma unroll
                for (int i = 0; i < R; i += 4) {
                    if (c0 + i < c1) {
                        const f32x4 v = *reinterpret_cast<const f32x4*>(L + c0 + i);
#pragma unroll
                        for (int e = 0; e < 4; ++e) u[i + e] = c0 + i + e < c1 ? order_key(v[e]) : 0u;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) u[i + e] = 0u;
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < R; ++i) u[i] = c0 + i < c1 ? order_key(L[c0 + i]) : 0u;
            }
        }
    }
    template <class F>
    __device__ void each(F f) const {
        if (R > 0) {
#pragma unroll
            for (int i = 0; i < R; ++i)
                if (c0 + i < c1) f(c0 + i, u[i]);
        } else {
            for (int i = c0; i < c1; ++i) f(i, order_key(L[i]));
        }
    }
};

template <int R>
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs p) {
    __shared__ uint32_t hist[2][kCopies][256];
    __shared__ uint32_t wsum[kWaves];
    __shared__ uint32_t red[2][kWaves];
    __shared__ uint32_t sel_digit, sel_above;
    const int r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = visible_entries(p.row_pos[r], p.m);
    const int k = p.k;
    int32_t* out = p.idx + (int64_t)r * k;
    if (n <= k) {
        for (int i = tid; i < k; i += kThreads) out[i] = i < n ? i : -1;
        return;
    }
    const int per_thread = ((n + kThreads - 1) / kThreads + 3) & ~3;
    Chunk<R> C;
    const float* row = p.logits + (int64_t)r * p.ld;
    C.init(row, n, per_thread, (reinterpret_cast<uintptr_t>(row) & 15) == 0);

    // 1. common leading bits of all keys
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    C.each([&](int, uint32_t u) { kmin = min(kmin, u); kmax = max(kmax, u); });
    for (int o = 32; o > 0; o >>= 1) {
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    }
    if (lane == 0) { red[0][wave] = kmin; red[1][wave] = kmax; }
    __syncthreads();
    kmin = red[0][0]; kmax = red[1][0];
    for (int i = 1; i < kWaves; ++i) { kmin = min(kmin, red[0][i]); kmax = max(kmax, red[1][i]); }
    const uint32_t diff = kmin ^ kmax;
    int top = diff ? 31 - __builtin_clz(diff) : -1;            // highest differing bit
    uint32_t mask = diff == 0 ? 0xffffffffu : top >= 31 ? 0u : ~((2u << top) - 1u);   // the common bits
    uint32_t prefix = kmax & mask;
    uint32_t need = (uint32_t)k;                                // keys still to take among those matching

    // 2. radix passes from the highest differing bit down.  Two histogram
    // buffers: while wave 0 sums the copies of this pass's buffer and scans
    // it, the other waves clear the buffer of the next pass.
    for (int i = tid; i < kCopies * 256; i += kThreads) (&hist[0][0][0])[i] = 0u;
    __syncthreads();
    int cur = 0;
    while (top >= 0) {
        const int w = min(8, top + 1);
        const int shift = top - w + 1;
        const uint32_t bins = 1u << w;
        uint32_t* h = hist[cur][lane & (kCopies - 1)];
        C.each([&](int, uint32_t u) {
            if ((u & mask) == prefix) atomicAdd(&h[(u >> shift) & (bins - 1)], 1u);
        });
        __syncthreads();
        if (tid < 64) {
            // lane l owns bins 4l..4l+3; suffix sums from the top digit down
            uint32_t c[4], s = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t t = 0;
#pragma unroll
                for (int cp = 0; cp < kCopies; ++cp) t += hist[cur][cp][4 * tid + i];
                c[i] = t;
                s += t;
            }
            uint32_t suf = s;
            for (int o = 1; o < 64; o <<= 1) {
                uint32_t t = __shfl_down(suf, o);
                if (tid + o < 64) suf += t;
            }
            uint32_t above = suf - s;        // keys in bins of higher lanes
#pragma unroll
            for (int i = 3; i >= 0; --i) {
                if (above < need && above + c[i] >= need) { sel_digit = 4 * tid + i; sel_above = above; }
                above += c[i];
            }
        } else {
            for (int i = tid - 64; i < kCopies * 256; i += kThreads - 64) (&hist[cur ^ 1][0][0])[i] = 0u;
        }
        __syncthreads();
        prefix |= sel_digit << shift;
        mask |= (bins - 1u) << shift;
        need -= sel_above;
        top = shift - 1;
        cur ^= 1;
    }
    const uint32_t T = prefix;

    // 3. ordered output
    uint32_t gt = 0, eq = 0;
    C.each([&](int, uint32_t u) { gt += u > T; eq += u == T; });
    uint32_t total;
    const uint32_t gt_before = block_exclusive_scan(gt, wsum, &total);
    const uint32_t eq_before = block_exclusive_scan(eq, wsum, &total);
    uint32_t pos = gt_before + min(eq_before, need);
    uint32_t eq_seen = eq_before;
    C.each([&](int i, uint32_t u) {
        if (u > T) out[pos++] = i;
        else if (u == T) {
            if (eq_seen < need) out[pos++] = i;
            ++eq_seen;
        }
    });
}

}  // namespace

hipError_t launch_topk_select(const TopkArgs& a, int max_entries, hipStream_t stream) {
    if (a.num_rows <= 0 || a.k <= 0) return hipSuccess;
    const int per_thread = ((max_entries + kThreads - 1) / kThreads + 3) & ~3;
    if (per_thread <= 8) hipLaunchKernelGGL(topk_kernel<8>, dim3(a.num_rows), dim3(kThreads), 0, stream, a);
    else if (per_thread <= 16) hipLaunchKernelGGL(topk_kernel<16>, dim3(a.num_rows), dim3(kThreads), 0, stream, a);
    else if (per_thread <= 32) hipLaunchKernelGGL(topk_kernel<32>, dim3(a.num_rows), dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL(topk_kernel<0>, dim3(a.num_rows), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lcca
