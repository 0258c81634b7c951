// topk_select: for each query row, the k visible entries with the largest
// indexer logits (equal logits: smaller entry first), written in ascending
// entry order and padded with -1.  [P1 = page "vLLM uveo DeepSeek V4 s 8,7x
// manjim KV cacheom", section "Kako funkcionira optimizacija KV cachea?":
// attention is limited to the top-k compressed tokens.]
//
// One 1024-thread workgroup per row.  Logits map to order-preserving u32
// keys (-0.0 folded onto +0.0); four 8-bit radix passes with LDS histograms
// find the k-th largest key T and how many keys equal to T are still
// needed; a final pass in index order keeps every key > T and the first
// `need` keys == T, with block-wide exclusive scans giving each kept entry
// its output slot, so the result is deterministic and sorted by entry.
#include "device.h"
#include "kernels.h"

namespace lcca {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

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

__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs p) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t wsum[kWaves];
    __shared__ uint32_t sel_digit, sel_above;
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int n = visible_entries(p.row_pos[r], p.m);
    const int k = p.k;
    int32_t* out = p.idx + (int64_t)r * k;
    if (n <= k) {
        for (int i = tid; i < k; i += kThreads) out[i] = i < n ? i : -1;
        return;
    }
    const float* L = p.logits + (int64_t)r * p.ld;

    uint32_t prefix = 0, mask = 0;
    uint32_t need = (uint32_t)k;            // keys still to take among those matching prefix
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kThreads) {
            uint32_t u = order_key(L[i]);
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            // lane l owns bins 4l..4l+3; suffix sums from the top digit down
            uint32_t c[4], s = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) { c[i] = hist[4 * tid + i]; s += c[i]; }
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
        }
        __syncthreads();
        prefix |= sel_digit << shift;
        mask |= 255u << shift;
        need -= sel_above;
        __syncthreads();
    }
    const uint32_t T = prefix;

    // final pass: contiguous chunk per thread, in entry order
    const int chunk = (n + kThreads - 1) / kThreads;
    const int c0 = min(tid * chunk, n), c1 = min(c0 + chunk, n);
    uint32_t gt = 0, eq = 0;
    for (int i = c0; i < c1; ++i) {
        uint32_t u = order_key(L[i]);
        gt += u > T;
        eq += u == T;
    }
    uint32_t tot;
    const uint32_t gt_before = block_exclusive_scan(gt, wsum, &tot);
    const uint32_t eq_before = block_exclusive_scan(eq, wsum, &tot);
    uint32_t pos = gt_before + min(eq_before, need);
    uint32_t eq_seen = eq_before;
    for (int i = c0; i < c1; ++i) {
        uint32_t u = order_key(L[i]);
        if (u > T) out[pos++] = i;
        else if (u == T) {
            if (eq_seen < need) out[pos++] = i;
            ++eq_seen;
        }
    }
}

}  // namespace

hipError_t launch_topk_select(const TopkArgs& a, int /*max_entries*/, hipStream_t stream) {
    if (a.num_rows <= 0 || a.k <= 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel, dim3(a.num_rows), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lcca
