// topk_select: for each query row, the k visible entries with the largest
// indexer logits (equal logits: smaller entry first), written in ascending
// entry order and padded with -1.  [Page "vLLM uveo DeepSeek V4 s 8,7x manjim
// KV cacheom", section "Kako funkcionira optimizacija KV cachea?": attention is
// limited to the top-k compressed tokens.]
//
// One 1024-thread workgroup per row.  Logits map to order-preserving u32 keys
// (-0.0 folded onto +0.0).  Thread t owns the 4-entry groups t, t + 1024,
// t + 2048, ... of the row, so every load is a coalesced 16-byte access.
// Rows of up to 32K entries are held in registers as full keys, rows of up
// to 128K as their leading 16 bits (two per register); longer rows are read
// again for each pass over them.
//   1. Histogram of the leading 12 key bits (sign, exponent, 3 mantissa
//      bits) in LDS; a block scan from the top bin finds the bin holding the
//      k-th largest key and how many keys lie above it.  In the fused decode
//      launch the indexer has already counted the row's keys per leading
//      digit; the selection loads those counts (and clears them) instead.
//   2. One pass marks every key of a higher bin in a bitmap of the row
//      (each 8-lane group assembles its 32-bit word with DPP moves and
//      stores it, no atomics) and collects the keys of the boundary bin,
//      with their entries, in LDS.
//   3. Radix passes over those candidates alone (bits 19..12, 11..4, 3..0)
//      give the k-th largest key T and how many keys equal to T are needed.
//      If the boundary bin overflows the candidate buffer, the same passes
//      run over the whole row instead.
//   4. Candidates above T join the bitmap; candidates equal to T go to a
//      second bitmap.  A block scan of the bitmaps' popcounts gives every
//      thread its output offset, so the result comes out sorted by entry and
//      the first `need` equal keys (smallest entries) are the ones kept.
// The leading-digit histogram keeps copies of every bin side by side
// ([bin][copy], the copy picked by lane), so lanes that hit the same bin land
// in different banks; the copies are summed into one count per bin before the
// scan, which then reads 4 consecutive bins per thread.  The full layout
// keeps 8 copies and bitmaps for 2^18 entries (~148 KB of LDS); the compact
// layout, for rows of up to 32K entries, 2 copies and bitmaps for 32K
// entries (~60 KB), which lets two rows share a compute unit and clears and
// sums a quarter of the copies.
#include "compress_dev.h"
#include "device.h"
#include "kernels.h"

namespace lcca {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kGroup = 4 * kThreads;            // entries per load round
constexpr int kLeadBits = kTopkLeadBits;
constexpr int kLeadShift = 32 - kLeadBits;
constexpr int kLeadBins = 1 << kLeadBits;
constexpr int kLeadCopies = 8;                  // lane & 7 picks the copy
constexpr int kCandCap = 4096;
constexpr int kWords = kTopkMaxEntries / 32;

// Shared memory of one row's selection.  The full layout (8 histogram copies,
// bitmaps for 2^18 entries) takes ~148 KB, one workgroup per compute unit;
// the compact one (2 copies, bitmaps for 32K entries) ~58 KB, so two rows
// share a compute unit when a launch has more rows than compute units.
template <int COPIES, int WORDS>
struct alignas(16) SmemT {
    union alignas(16) {
        uint32_t lead[kLeadBins * COPIES];            // step 1: [bin][copy]
        struct {
            uint32_t bits[2][WORDS];                  // [0] keys above T, [1] keys equal to T
            union alignas(16) {
                struct {
                    uint32_t key[kCandCap];
                    int32_t idx[kCandCap];
                } c;                                  // the boundary digit's candidates
                uint32_t sel[2 * kCandCap];           // later: the selected positions, in output order
            } cs;
            uint32_t fine[2][256];                    // refinement histograms, double-buffered
        } b;
    } u;
    alignas(16) uint32_t cnt[kLeadBins];              // step 1: copies summed
    uint32_t wsum[2][kWaves];
    uint32_t cand_n, sel_digit, sel_above;
};
constexpr int kCompactEntries = 32768;

// OR of x over each aligned group of 8 lanes (DPP: swap within pairs, within
// quads, then mirror the two quads of the group).
__device__ inline uint32_t or8(uint32_t x) {
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false);   // row_half_mirror
    return x;
}

// Inclusive prefix sum over the wave (DPP: shifts within rows of 16 lanes,
// then row broadcasts of lanes 15 and 31).
__device__ inline uint32_t wave_incl_sum(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);   // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return x;
}

// Exclusive scans of a and b over the block, in thread order.
__device__ inline void block_exclusive_scan2(uint32_t& a, uint32_t& b, uint32_t (*wsum)[kWaves]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t ia = wave_incl_sum(a), ib = wave_incl_sum(b);
    __syncthreads();
    if (lane == 63) { wsum[0][w] = ia; wsum[1][w] = ib; }
    __syncthreads();
    uint32_t ba = 0, bb = 0;
    for (int i = 0; i < w; ++i) { ba += wsum[0][i]; bb += wsum[1][i]; }
    a = ba + ia - a;
    b = bb + ib - b;
}

// The row's keys.  R > 0: R keys per thread in registers, full (Half false)
// or their leading 16 bits (Half true, two per register); R == 0: read from
// memory on every pass.  Vec: every row starts 16-byte aligned, so a 4-entry
// group is one 16-byte load (the row holds ld >= n floats, and the last
// group's load is clamped to the last group that starts below n).  Loads
// are branch-free: addresses are clamped into the row and entries >= n
// masked.
template <int R, bool Half, bool Vec, bool U>
struct Keys {
    static constexpr int kRounds = R / 4;
    static constexpr bool kFull = R > 0 && !Half;      // full keys without memory reads
    uint32_t u[R == 0 ? 1 : (Half ? R / 2 : R)];
    const float* L;                                    // logits (U false) or order keys (U true)
    int n, rounds;

    __device__ __forceinline__ static uint32_t key_of(uint32_t bits) {
        return U ? bits : order_key(__uint_as_float(bits));
    }
    __device__ __forceinline__ void load4(int e, uint32_t* o) const {
        const uint32_t* B = reinterpret_cast<const uint32_t*>(L);
        if constexpr (Vec) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(B + min(e, (n - 1) & ~3));
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = e + i < n ? key_of(v[i]) : 0u;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t x = B[min(e + i, n - 1)];
                o[i] = e + i < n ? key_of(x) : 0u;
            }
        }
    }
    // First entry of the thread's group in round j.  Every pass takes its
    // own opaque copy of the thread index, so entry offsets are recomputed
    // per pass rather than kept live (or spilled) across the whole kernel.
    __device__ __forceinline__ static int tid_copy() {
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        return t;
    }
    __device__ __forceinline__ static int first(int t, int j) { return 4 * (t + kThreads * j); }

    __device__ __forceinline__ void init(const float* row, int n_) {
        L = row; n = n_;
        rounds = (n + kGroup - 1) / kGroup;
        if constexpr (R > 0) {
            const int t = tid_copy();
            constexpr int kBatch = kRounds < (Half ? 4 : 8) ? kRounds : (Half ? 4 : 8);
#pragma unroll
            for (int j0 = 0; j0 < kRounds; j0 += kBatch) {
                uint32_t v[kBatch][4];
#pragma unroll
                for (int b = 0; b < kBatch; ++b) load4(first(t, j0 + b), v[b]);
#pragma unroll
                for (int b = 0; b < kBatch; ++b) {
                    if constexpr (Half) {
                        u[2 * (j0 + b)] = (v[b][0] >> 16) | (v[b][1] & 0xffff0000u);
                        u[2 * (j0 + b) + 1] = (v[b][2] >> 16) | (v[b][3] & 0xffff0000u);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) u[4 * (j0 + b) + i] = v[b][i];
                    }
                }
                // at most one batch of loads in flight per thread
                if constexpr (Half) __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    // f(first entry of the thread's group, its 4 keys) once per round, the
    // same number of calls in every thread; entries >= n must be skipped by
    // f.  With Half the keys carry their leading 16 bits only.
    template <class F>
    __device__ __forceinline__ void rounds_each(F f) const {
        if constexpr (R > 0) {
            const int t = tid_copy();
#pragma unroll
            for (int j = 0; j < kRounds; ++j) {
                if (j < rounds) {
                    uint32_t k[4];
                    if constexpr (Half) {
                        k[0] = u[2 * j] << 16; k[1] = u[2 * j] & 0xffff0000u;
                        k[2] = u[2 * j + 1] << 16; k[3] = u[2 * j + 1] & 0xffff0000u;
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) k[i] = u[4 * j + i];
                    }
                    f(first(t, j), k);
                    // keep the scheduler from hoisting later rounds' work
                    // (and their registers) above this one
                    if constexpr (Half) __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
            stream_rounds(f);
        }
    }
    template <class F>
    __device__ __forceinline__ void stream_rounds(F f) const {
        const int t = tid_copy();
        for (int j = 0; j < rounds; j += 2) {
            uint32_t t0[4], t1[4];
            const int e0 = first(t, j), e1 = e0 + kGroup;
            load4(e0, t0);
            if (j + 1 < rounds) load4(e1, t1);
            f(e0, t0);
            if (j + 1 < rounds) f(e1, t1);
        }
    }
    // f(entry, full key) for every entry < n
    template <class F>
    __device__ __forceinline__ void each_full(F f) const {
        auto g = [&](int e, const uint32_t* k) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (e + i < n) f(e + i, k[i]);
        };
        if constexpr (kFull) rounds_each(g);
        else stream_rounds(g);
    }
    __device__ __forceinline__ uint32_t full_key(int e, uint32_t k) const {
        if constexpr (kFull) return k;
        else return key_of(reinterpret_cast<const uint32_t*>(L)[e]);
    }
};

// Wave 0 reads the 256-bin histogram `h` (lane l: bins 4l .. 4l+3) and finds
// the digit holding the need-th largest key among those counted.
__device__ __forceinline__ void pick_digit(const uint32_t* h, uint32_t need, uint32_t* sel_digit, uint32_t* sel_above) {
    const int lane = threadIdx.x;
    const u32x4 v = *reinterpret_cast<const u32x4*>(h + 4 * lane);
    uint32_t c[4] = {v[0], v[1], v[2], v[3]};
    const uint32_t s = c[0] + c[1] + c[2] + c[3];
    const uint32_t incl = wave_incl_sum(s);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    uint32_t above = total - incl;            // keys in the bins of higher lanes
#pragma unroll
    for (int i = 3; i >= 0; --i) {
        if (above < need && above + c[i] >= need) { *sel_digit = 4 * lane + i; *sel_above = above; }
        above += c[i];
    }
}

// Radix passes over the keys `each` enumerates that match `prefix` under
// `mask`, from bit `top` down; leaves the need-th largest key in *prefix and
// the number of keys equal to it still needed in *need.  fine[0] must be
// zero on entry.
template <class SM, class Each>
__device__ __forceinline__ void refine(SM& sm, Each each, int top, uint32_t* prefix_io, uint32_t* mask_io, uint32_t* need_io) {
    const int tid = threadIdx.x;
    uint32_t prefix = *prefix_io, mask = *mask_io, need = *need_io;
    int cur = 0;
    while (top >= 0) {
        const int w = min(8, top + 1);
        const int shift = top - w + 1;
        const uint32_t bins = 1u << w;
        uint32_t* h = sm.u.b.fine[cur];
        each([&](int, uint32_t key) __attribute__((always_inline)) {
            if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & (bins - 1)], 1u);
        });
        __syncthreads();
        if (tid < 64) {
            pick_digit(h, need, &sm.sel_digit, &sm.sel_above);
        } else {
            if (tid < 128) reinterpret_cast<u32x4*>(sm.u.b.fine[cur ^ 1])[tid - 64] = u32x4{0u, 0u, 0u, 0u};
        }
        __syncthreads();
        prefix |= sm.sel_digit << shift;
        mask |= (bins - 1u) << shift;
        need -= sm.sel_above;
        top = shift - 1;
        cur ^= 1;
        // sel_digit is rewritten only after the next pass's first barrier,
        // which every thread reaches after reading it here
    }
    *prefix_io = prefix; *mask_io = mask; *need_io = need;
}

// What a selection reads and where its result goes.
//   kRow:   one row's logits -> topk_idx[r][0..k), ascending entries.
//   kSlice: slice s of row r (entries [s*L, (s+1)*L)) -> its own top-k as
//           candidates (order key, entry) in the workspace, ascending
//           entries, padded with (0, -1).
//   kCand:  the candidates of all slices of row r, whose positions ascend
//           with the entries (slice-major), -> topk_idx[r] (the entries
//           behind the selected positions).  Equal keys: smaller position,
//           i.e. smaller entry, first.
enum Mode : int { kRow = 0, kSlice = 1, kCand = 2 };

// The selection of row r (slice `by` of it in kSlice mode) by one workgroup.
template <int R, bool Half, bool Vec, int MODE, bool COMPACT>
__device__ __forceinline__ void topk_body(const TopkArgs& p, int r, int by) {
    static_assert(!COMPACT || (R > 0 && R <= 32 && !Half), "compact layout: rows of up to 32K entries in registers");
    constexpr int COPIES = COMPACT ? 2 : kLeadCopies;
    __shared__ SmemT<COPIES, COMPACT ? kCompactEntries / 32 : kWords> sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int n_row = visible_entries(checked(p.row_pos[r], 0, p.max_pos, p.dbg, kDbgRow), p.m);
    const int k = p.k;
    int32_t* out = p.idx + (int64_t)r * k;
    const int s0 = MODE == kSlice ? by * p.slice_len : 0;
    const int64_t c0 = (int64_t)r * p.cand_stride + (MODE == kSlice ? (int64_t)by * k : 0);
    int n;
    const float* base;
    if constexpr (MODE == kRow) {
        n = n_row;
        base = p.logits + (int64_t)r * p.ld;
    } else if constexpr (MODE == kSlice) {
        n = max(0, min(n_row - s0, p.slice_len));
        base = p.logits + (int64_t)r * p.ld + s0;
    } else {
        n = p.nslices * k;
        base = reinterpret_cast<const float*>(p.cand_key + c0);
    }
    // leading-digit counts of this row from the indexer (fused decode launch).
    // kRow: the row's own counts.  kSlice: the whole row's counts, read by
    // every slice of the row; with them a slice keeps its keys above the
    // row's boundary digit and, of its keys in that digit, the `need` largest
    // (at most k entries, the rest of its slots padded), so every entry of the
    // row's top-k survives.  kCand: the same counts again; the candidates
    // hold every key of the row above the boundary digit and at least `need`
    // of its keys in it, so the boundary digit and the count above it are the
    // row's.  kRow and kCand clear the counts once read (the clearing store
    // is issued only after the counts have arrived).
    u32x4* const hist = p.lead_hist ? reinterpret_cast<u32x4*>(p.lead_hist + (int64_t)r * kLeadBins) : nullptr;
    constexpr bool kClearCounts = MODE != kSlice;
    u32x4 hist_v = u32x4{0u, 0u, 0u, 0u};
    if (hist) hist_v = hist[tid];
    if (MODE == kSlice ? n <= k : n_row <= k) {
        if (hist && kClearCounts) {
            asm volatile("" ::"v"(hist_v[0]) : "memory");        // the counts have arrived
            hist[tid] = u32x4{0u, 0u, 0u, 0u};
        }
        if constexpr (MODE == kSlice) {
            for (int i = tid; i < k; i += kThreads) {
                p.cand_key[c0 + i] = i < n ? order_key(base[i]) : 0u;
                p.cand_idx[c0 + i] = i < n ? s0 + i : -1;
            }
        } else {
            for (int i = tid; i < k; i += kThreads) out[i] = i < n_row ? i : -1;
        }
        return;
    }
    // the selected position `e` at output slot `pos`.  kSlice and kCand
    // outputs need a load per selected position (its logit, its entry): with
    // up to kStageCap slots the positions are staged in LDS (over the
    // candidate arrays, free by then) and translated after one barrier, all
    // loads in flight together, instead of one dependent load per emitted
    // position in the bit loop.
    static constexpr int kStageCap = 2 * kCandCap;          // slots of sm.u.b.cs.sel
    const bool staged = MODE != kRow && k <= kStageCap;
    auto emit = [&](uint32_t pos, int e) __attribute__((always_inline)) {
        if (pos >= (uint32_t)k) return;                // never taken; keeps every store in the row
        if constexpr (MODE == kRow) {
            out[pos] = e;
        } else {
            if (staged) {
                sm.u.b.cs.sel[pos] = (uint32_t)e;
                return;
            }
            if constexpr (MODE == kSlice) {
                p.cand_key[c0 + pos] = order_key(base[e]);
                p.cand_idx[c0 + pos] = s0 + e;
            } else {
                out[pos] = p.cand_idx[c0 + e];
            }
        }
    };
    Keys<R, Half, Vec, MODE == kCand> K;
    K.init(base, n);

    if (hist) {
        // 1. the counts the indexer took (4096 bins = 1024 threads x 4)
        static_assert(kLeadBins == 4 * kThreads, "one 16-byte chunk of counts per thread");
        reinterpret_cast<u32x4*>(sm.cnt)[tid] = hist_v;
        if constexpr (kClearCounts) {
            asm volatile("" ::"v"(hist_v[0]) : "memory");        // the counts have arrived
            hist[tid] = u32x4{0u, 0u, 0u, 0u};
        }
        if (tid == 0) sm.cand_n = 0;
        __syncthreads();
    } else {
    {
        u32x4* z = reinterpret_cast<u32x4*>(sm.u.lead);
        for (int i = tid; i < kLeadBins * COPIES / 4; i += kThreads) z[i] = u32x4{0u, 0u, 0u, 0u};
    }
    if (tid == 0) sm.cand_n = 0;
    __syncthreads();

    // 1. leading-digit histogram and the boundary bin
    {
        const int copy = lane & (COPIES - 1);
        K.rounds_each([&](int e, const uint32_t* key) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                atomicAdd(&sm.u.lead[(key[i] >> kLeadShift) * COPIES + copy], e + i < n ? 1u : 0u);
        });
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kLeadBins * COPIES / 4 / kThreads; ++i) {
        const int chunk = tid + kThreads * i;
        const u32x4 x = reinterpret_cast<const u32x4*>(sm.u.lead)[chunk];
        if constexpr (COPIES == 8) {
            // lane pairs read one bin's 8 copies as two consecutive 16-byte
            // chunks and add them across the pair
            uint32_t c = x[0] + x[1] + x[2] + x[3];
            c += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)c, 0xB1, 0xF, 0xF, false);     // quad_perm [1,0,3,2]
            if ((chunk & 1) == 0) sm.cnt[chunk >> 1] = c;
        } else {
            // a 16-byte chunk holds the 2 copies of two bins
            static_assert(COPIES == 2, "copies");
            sm.cnt[2 * chunk] = x[0] + x[1];
            sm.cnt[2 * chunk + 1] = x[2] + x[3];
        }
    }
    __syncthreads();
    }
    {
        // thread t owns bins 4095-4t .. 4092-4t, so thread order is descending bins
        const u32x4 v = *reinterpret_cast<const u32x4*>(&sm.cnt[kLeadBins - 4 - 4 * tid]);
        const uint32_t c[4] = {v[3], v[2], v[1], v[0]};
        const uint32_t s = c[0] + c[1] + c[2] + c[3];
        uint32_t above = s, unused = 0;
        block_exclusive_scan2(above, unused, sm.wsum);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (above < (uint32_t)k && above + c[i] >= (uint32_t)k) {
                sm.sel_digit = kLeadBins - 1 - 4 * tid - i;
                sm.sel_above = above;
            }
            above += c[i];
        }
    }
    __syncthreads();
    const uint32_t lead = sm.sel_digit;
    uint32_t need = (uint32_t)k - sm.sel_above;
    __syncthreads();                          // the histogram's LDS is reused from here on

    // 2. bitmap of the keys above the boundary bin; candidates of the bin
    const int W = (n + 31) / 32;
    if (tid < 64) reinterpret_cast<u32x4*>(sm.u.b.fine[0])[tid] = u32x4{0u, 0u, 0u, 0u};
    auto words = [&](int e, const uint32_t* key, uint32_t& ncand) __attribute__((always_inline)) {
        uint32_t above = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t d = key[i] >> kLeadShift;
            above |= (d > lead && e + i < n ? 1u : 0u) << i;
            ncand += d == lead && e + i < n ? 1u : 0u;
        }
        const uint32_t word = or8(above << (4 * (lane & 7)));
        const int wi = e >> 5;
        if ((lane & 7) == 0 && wi < W) { sm.u.b.bits[0][wi] = word; sm.u.b.bits[1][wi] = 0u; }
    };
    auto put = [&](uint32_t c, int e, uint32_t key) __attribute__((always_inline)) {
        if (c < (uint32_t)kCandCap) {
            if constexpr (Keys<R, Half, Vec, MODE == kCand>::kFull) sm.u.b.cs.c.key[c] = key;
            sm.u.b.cs.c.idx[c] = e;
        }
    };
    if constexpr (R > 0) {
        // count this thread's candidates, reserve their slots with one LDS
        // atomic per wave, then write them
        uint32_t mine = 0;
        K.rounds_each([&](int e, const uint32_t* key) __attribute__((always_inline)) { words(e, key, mine); });
        const uint32_t incl = wave_incl_sum(mine);
        uint32_t base = 0;
        if (lane == 63 && incl > 0) base = atomicAdd(&sm.cand_n, incl);
        uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)base, 63) + incl - mine;
        if (mine > 0) {
            K.rounds_each([&](int e, const uint32_t* key) __attribute__((always_inline)) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if ((key[i] >> kLeadShift) == lead && e + i < n) put(c++, e + i, key[i]);
            });
        }
    } else {
        K.rounds_each([&](int e, const uint32_t* key) __attribute__((always_inline)) {
            uint32_t unused = 0;
            words(e, key, unused);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if ((key[i] >> kLeadShift) == lead && e + i < n) put(atomicAdd(&sm.cand_n, 1u), e + i, key[i]);
        });
    }
    __syncthreads();

    // 3. the k-th largest key within the boundary bin
    const uint32_t nc = sm.cand_n;
    uint32_t T = lead << kLeadShift, mask = ~0u << kLeadShift;
    const bool fits = nc <= (uint32_t)kCandCap;
    if constexpr (!Keys<R, Half, Vec, MODE == kCand>::kFull) {
        if (fits) {
            for (int c = tid; c < (int)nc; c += kThreads) sm.u.b.cs.c.key[c] = K.full_key(sm.u.b.cs.c.idx[c], 0u);
            __syncthreads();
        }
    }
    auto cands = [&](auto f) __attribute__((always_inline)) {
        for (int c = tid; c < (int)nc; c += kThreads) f(sm.u.b.cs.c.idx[c], sm.u.b.cs.c.key[c]);
    };
    auto row_bin = [&](auto f) __attribute__((always_inline)) {
        K.each_full([&](int e, uint32_t key) __attribute__((always_inline)) {
            if ((key >> kLeadShift) == lead) f(e, key);
        });
    };
    if (MODE == kSlice && hist && nc <= need) {
        // a slice with no more keys in the row's boundary digit than the row
        // needs from it keeps them all
        need = nc;
    } else if (fits) {
        refine(sm, cands, kLeadShift - 1, &T, &mask, &need);
    } else {
        refine(sm, row_bin, kLeadShift - 1, &T, &mask, &need);
    }

    // 4. keys of the bin above T or equal to it join the bitmaps
    auto mark = [&](int e, uint32_t key) __attribute__((always_inline)) {
        if (key > T) atomicOr(&sm.u.b.bits[0][e >> 5], 1u << (e & 31));
        else if (key == T) atomicOr(&sm.u.b.bits[1][e >> 5], 1u << (e & 31));
    };
    if (fits) cands(mark);
    else row_bin(mark);
    __syncthreads();

    const int wpt = (W + kThreads - 1) / kThreads;
    const int w0 = min(W, tid * wpt), w1 = min(W, w0 + wpt);
    uint32_t gt = 0, eq = 0;
    for (int w = w0; w < w1; ++w) { gt += __popc(sm.u.b.bits[0][w]); eq += __popc(sm.u.b.bits[1][w]); }
    block_exclusive_scan2(gt, eq, sm.wsum);
    uint32_t pos = gt + min(eq, need);
    uint32_t eq_seen = eq;
    for (int w = w0; w < w1; ++w) {
        const uint32_t g = sm.u.b.bits[0][w], q = sm.u.b.bits[1][w];
        uint32_t any = g | q;
        while (any) {
            const int b = __builtin_ctz(any);
            any &= any - 1;
            const int e = 32 * w + b;
            const bool take = ((g >> b) & 1u) || eq_seen < need;
            eq_seen += (g >> b) & 1u ? 0u : 1u;
            if (take) emit(pos++, e);
        }
    }
    if constexpr (MODE != kRow) {
        // the last thread's end position is the number kept
        if (staged || (MODE == kSlice && hist)) {
            __syncthreads();
            if (tid == kThreads - 1) sm.cand_n = pos;
            __syncthreads();
        }
        if (staged) {
            const uint32_t* sel = sm.u.b.cs.sel;
            for (int i = tid; i < (int)sm.cand_n; i += kThreads) {
                const int e = (int)sel[i];
                if constexpr (MODE == kSlice) {
                    p.cand_key[c0 + i] = order_key(base[e]);
                    p.cand_idx[c0 + i] = s0 + e;
                } else {
                    out[i] = p.cand_idx[c0 + e];
                }
            }
        }
        if constexpr (MODE == kSlice) {
            if (hist) {
                // pad the slice's slots past the number kept
                for (int i = (int)sm.cand_n + tid; i < k; i += kThreads) {
                    p.cand_key[c0 + i] = 0u;
                    p.cand_idx[c0 + i] = -1;
                }
            }
        }
    }
}

template <int R, bool Half, bool Vec, int MODE, bool COMPACT>
__global__ __launch_bounds__(kThreads, COMPACT ? 8 : 4) void topk_kernel(TopkArgs p) {
    topk_body<R, Half, Vec, MODE, COMPACT>(p, blockIdx.x, blockIdx.y);
}

// One decode launch holding the rows' one-launch top-k selections (kRow) or
// the selections among their slices' candidates (kCand) in workgroups
// 0 .. rows-1 with the compact layout, and, on the compute units they leave
// idle, compress_append of the step's new tokens: workgroup rows + i runs
// item i of compress_append's (token, slice) grid on its first four waves
// (the other waves exit at once, so its barriers count the four).  Nothing
// the selections read is written by compress_append.
template <int R, int MODE, int TOK>
__global__ __launch_bounds__(kThreads) void topk_compress_kernel(TopkArgs p, CompressArgs c, int items) {
    const int w = (int)blockIdx.x;
    if (w < p.num_rows) {
        topk_body<R, false, true, MODE, true>(p, w, 0);
        return;
    }
    if ((int)threadIdx.x >= cmp::kThreads) return;
    const int it = w - p.num_rows;
    cmp::compress_append_body<TOK>(c, it / items, it % items);
}

template <int R, bool Vec, int MODE>
void launch_regs(const TopkArgs& a, bool compact, dim3 grid, hipStream_t stream) {
    if (compact) hipLaunchKernelGGL((topk_kernel<R, false, Vec, MODE, true>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((topk_kernel<R, false, Vec, MODE, false>), grid, dim3(kThreads), 0, stream, a);
}

// One-launch selections of rows of up to 32K entries use the compact layout
// when the launch has more rows than the GPU has compute units (256: two rows
// per compute unit hide each other's barriers) or at most 64 rows (clearing
// and summing two histogram copies instead of eight is then the gain).  In
// between, two rows per compute unit could leave compute units idle, and the
// two-launch path keeps eight copies: its candidate keys are concentrated, so
// two copies conflict more (lp_512k: 33.9 against 35.6 us).
template <bool Vec, int MODE>
void launch_sel(const TopkArgs& a, int entries, dim3 grid, hipStream_t stream) {
    const int rounds = (entries + kGroup - 1) / kGroup;
    const dim3 block(kThreads);
    const int64_t wgs = (int64_t)grid.x * grid.y;
    const bool compact = MODE == kRow && (wgs > 256 || wgs <= 64);
    if (rounds <= 2) launch_regs<8, Vec, MODE>(a, compact, grid, stream);
    else if (rounds <= 4) launch_regs<16, Vec, MODE>(a, compact, grid, stream);
    else if (rounds <= 8) launch_regs<32, Vec, MODE>(a, compact, grid, stream);
    else if (rounds <= 32) hipLaunchKernelGGL((topk_kernel<128, true, Vec, MODE, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((topk_kernel<0, false, Vec, MODE, false>), grid, block, 0, stream, a);
}

}  // namespace

int topk_slices(int max_entries) {
    return max_entries > kTopkSplitAbove ? (max_entries - 1) / kTopkSlice + 1 : 1;
}

int64_t topk_cand_stride(int max_entries, int k) {
    return ((int64_t)topk_slices(max_entries) * k + 3) & ~(int64_t)3;
}

// Entries the compact-layout selection of the fused launch takes: the row
// itself (one launch) or its slices' candidates (two launches).
static int64_t fused_sel_entries(int max_entries, int k) {
    const int ns = topk_slices(max_entries);
    return ns == 1 ? (int64_t)max_entries : (int64_t)ns * k;
}

bool topk_compress_supported(const TopkArgs& a, int max_entries, int tok_dtype) {
    const bool vec = (reinterpret_cast<uintptr_t>(a.logits) & 15) == 0 && a.ld % 4 == 0;
    return vec && fused_sel_entries(max_entries, a.k) <= 8 * kGroup && tok_dtype == DT_BF16;
}

hipError_t launch_topk_compress(TopkArgs a, int max_entries, const CompressArgs& c, int total_new, hipStream_t stream) {
    if (!topk_compress_supported(a, max_entries, c.tok_dtype)) return hipErrorInvalidValue;
    const int SK = (c.D + cmp::kSliceDims - 1) / cmp::kSliceDims;
    const int SI = c.ik_data != nullptr ? (c.dI + cmp::kSliceDims - 1) / cmp::kSliceDims : 0;
    const int items = SK + SI + 1;
    const dim3 grid((unsigned)(a.num_rows + (int64_t)total_new * items)), block(kThreads);
    const int ns = topk_slices(max_entries);
    if (ns > 1) {
        // each slice's top-k first (as in launch_topk_select), then the
        // selection among the candidates beside compress_append
        a.nslices = ns;
        a.slice_len = kTopkSlice;
        launch_sel<true, kSlice>(a, kTopkSlice, dim3(a.num_rows, ns), stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int rounds = (int)((fused_sel_entries(max_entries, a.k) + kGroup - 1) / kGroup);
#define LCCA_TC(R)                                                                                         \
    if (ns == 1) hipLaunchKernelGGL((topk_compress_kernel<R, kRow, DT_BF16>), grid, block, 0, stream, a, c, items); \
    else hipLaunchKernelGGL((topk_compress_kernel<R, kCand, DT_BF16>), grid, block, 0, stream, a, c, items);
    if (rounds <= 2) { LCCA_TC(8) }
    else if (rounds <= 4) { LCCA_TC(16) }
    else { LCCA_TC(32) }
#undef LCCA_TC
    return hipGetLastError();
}

hipError_t launch_topk_select(TopkArgs a, int max_entries, hipStream_t stream) {
    if (a.num_rows <= 0 || a.k <= 0) return hipSuccess;
    const bool vec = (reinterpret_cast<uintptr_t>(a.logits) & 15) == 0 && a.ld % 4 == 0;
    const int ns = topk_slices(max_entries);
    if (ns == 1) {
        if (vec) launch_sel<true, kRow>(a, max_entries, dim3(a.num_rows), stream);
        else launch_sel<false, kRow>(a, max_entries, dim3(a.num_rows), stream);
        return hipGetLastError();
    }
    // long rows: each slice's top-k first, then the top-k of their candidates
    a.nslices = ns;
    a.slice_len = kTopkSlice;
    if (vec) launch_sel<true, kSlice>(a, kTopkSlice, dim3(a.num_rows, ns), stream);
    else launch_sel<false, kSlice>(a, kTopkSlice, dim3(a.num_rows, ns), stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_sel<true, kCand>(a, ns * a.k, dim3(a.num_rows), stream);
    return hipGetLastError();
}

}  // namespace lcca
