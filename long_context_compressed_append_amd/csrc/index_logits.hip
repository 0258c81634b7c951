// index_logits: sparse MQA logits of the indexer,
//     l[r][g] = s_I * sum_h w[r][h] * max(0, q[r][h] . K_g),  g < n_r,
// over the paged indexer-key pool.  [P3 = page "DeepSeek-V4.1-Flash ve vLLM:
// kde se vzala 5,3x vyssi propustnost", section "Vykon neprinesl jeden
// kernel": scores are computed only for candidate positions, here every
// causally visible entry and nothing beyond it.]
//
// bf16 path (MFMA 32x32x16): heads on M, entries on N, the head dim on K.
// Each wave keeps its row's query (HI x dI bf16) in VGPRs as A operands and
// streams 32-entry tiles of keys straight from HBM into B-operand registers
// (bf16 as stored; E4M3 converted exactly to bf16 in registers), with the
// next tile's loads in flight during the current tile's MFMAs.  The output
// C layout gives each lane 16 heads of one entry, so ReLU, the per-head
// weight and most of the head sum stay in registers; one cross-lane add
// finishes it.  The contraction's k order is a permutation shared by A and
// B: lane half g covers dims [g*dI/2, (g+1)*dI/2), 8 per k-step, so each lane
// reads dI contiguous bytes of its key.
//
// Decode (few rows): a workgroup covers one row, its 4 waves stream disjoint
// tile ranges.  Prefill (many rows): index_rows_kernel, eight rows per
// workgroup sharing key tiles staged in LDS.
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace lcca {

namespace {

constexpr int kThreads = 256;

// Raw key registers of one lane: its half of one entry's key, loaded as
// stored (bf16, or E4M3 converted to bf16 right before the MFMA), so a tile
// in flight costs 32 (bf16) or 16 (FP8) VGPRs.
template <int KD, int KS>
struct RawKey {
    typedef typename std::conditional<KD == DT_BF16, u32x4, u32x2>::type word;
    word w[KS];
};

template <int KD, int KS>
__device__ __forceinline__ void load_key(const uint8_t* keys, int64_t row, int g, RawKey<KD, KS>& k) {
    constexpr int DI = KS * 16, HALF = DI / 2;
    if constexpr (KD == DT_BF16) {
        const u32x4* src = reinterpret_cast<const u32x4*>(keys + (row * DI + g * HALF) * 2);
#pragma unroll
        for (int s = 0; s < KS; ++s) k.w[s] = src[s];
    } else {
        const u32x2* src = reinterpret_cast<const u32x2*>(keys + row * DI + g * HALF);
#pragma unroll
        for (int s = 0; s < KS; ++s) k.w[s] = src[s];
    }
}

template <int KD, int KS>
__device__ inline bf16x8 key_operand(const RawKey<KD, KS>& k, int s) {
    if constexpr (KD == DT_BF16) {
        return __builtin_bit_cast(bf16x8, k.w[s]);
    } else {
        return __builtin_bit_cast(bf16x8, fp8x8_to_bf16(k.w[s][0], k.w[s][1]));
    }
}

// FP8 keys as B operands of the 32x32x64 FP8 MFMA: a lane's 32-byte k-block
// s8 is bytes [32 s8, 32 s8 + 32) of the 64 contiguous bytes it loaded.
template <int KS>
__device__ inline i32x8 key_operand8(const RawKey<DT_FP8, KS>& k, int s8) {
    return i32x8{(int)k.w[4 * s8][0],     (int)k.w[4 * s8][1],     (int)k.w[4 * s8 + 1][0], (int)k.w[4 * s8 + 1][1],
                 (int)k.w[4 * s8 + 2][0], (int)k.w[4 * s8 + 2][1], (int)k.w[4 * s8 + 3][0], (int)k.w[4 * s8 + 3][1]};
}

// FP8 queries: each head's query row (bf16 in q_lds, rows of QROWB bytes)
// is quantised: X = floor(log2 max |q_h|) - 7 (the row maximum / 2^X lands
// in [128, 256), no saturation; X = -127 for a zero row), q8 = RNE E4M3 of
// q / 2^X.  The codes go to q8_lds (rows of Q8ROWB bytes), X to x_lds[h],
// and q_lds is overwritten with q8 * 2^X, which bf16 holds exactly.  All
// kThreads threads: head tid / P, part tid % P of P = kThreads / heads parts
// (adjacent lanes).
template <int NHT, int DI, int QROWB, int Q8ROWB>
__device__ void quantize_query_lds(uint8_t* q_lds, uint8_t* q8_lds, int* x_lds) {
    constexpr int NH = NHT * 32, P = kThreads / NH, DP = DI / P;
    static_assert(P >= 1 && (P & (P - 1)) == 0 && DP % 8 == 0, "query parts of whole 16-byte units");
    const int tid = threadIdx.x, h = tid / P, part = tid % P;
    uint16_t* row = reinterpret_cast<uint16_t*>(q_lds + h * QROWB) + part * DP;
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < DP; ++i) amax = fmaxf(amax, fabsf(bf16_to_f32(row[i])));
#pragma unroll
    for (int o = 1; o < P; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    int X = -127;
    if (amax > 0.0f) {
        int ex = 0;
        (void)frexpf(amax, &ex);
        X = min(max(ex - 1 - 7, -127), 127);
    }
    uint8_t* codes = q8_lds + h * Q8ROWB + part * DP;
#pragma unroll
    for (int i = 0; i < DP; ++i) {
        const uint32_t c = f32_to_fp8_inrange(ldexpf(bf16_to_f32(row[i]), -X));   // |.| < 256
        codes[i] = (uint8_t)c;
        row[i] = (uint16_t)f32_to_bf16(ldexpf(fp8_value(c), X));
    }
    if (part == 0) x_lds[h] = X;
}

template <int N>
struct IntC {
    static constexpr int value = N;
};

// Register sets of keys per wave (PF - 1 tiles in flight) at two waves per
// SIMD (the head weights are read from LDS per tile to make room): FP8
// waves (half the registers per tile) keep three tiles in flight, bf16
// waves one (two measured no faster).
template <int KD>
constexpr int key_depth() {
    return KD == DT_FP8 ? 4 : 2;
}
constexpr int kWavesPerSimd = 2;

// Calls f(IntC<J>, tile + J) for J = 0 .. PF-1 while tile + J < t_end.
template <int J, int PF, class F>
__device__ __forceinline__ void unroll_steps(F& f, int tile, int t_end) {
    if constexpr (J < PF) {
        if (tile + J < t_end) {
            f(IntC<J>{}, tile + J);
            unroll_steps<J + 1, PF>(f, tile, t_end);
        }
    }
}

// Inputs of the entry a row's own token completes (decode launches ahead of
// the step's compress_append, groups of m <= 4 tokens): lane i < m holds
// token i's logit; every lane holds its DI / 64 dimensions of the group's
// tokens as raw bits (bf16 or fp32); the earlier m - 1 tokens come from the
// remainder ring (slot i), the last is token r of the batch; and the
// sequence's cu_new and start_pos entries, which check that it is.
template <int DI>
struct FreshIn {
    static constexpr int DPL = DI / 64;                          // dimensions per lane
    float logit;
    uint32_t raw[4][DPL];
    int cu0, cu1, sp;                                            // cu_new[b], cu_new[b + 1], start_pos[b]

    __device__ __forceinline__ void load(const IndexArgs& p, int r, int b) {
        const int m = p.m, lane = threadIdx.x & 63;
        cu0 = p.cu_new[b];
        cu1 = p.cu_new[b + 1];
        sp = p.start_pos[b];
        logit = -INFINITY;
        if (lane < m) logit = lane == m - 1 ? p.ik_logit[r] : p.rem_ik_logit[(int64_t)b * m + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool last = i == m - 1;
            const void* base = last ? p.ik_tok : p.rem_ik;
            const int64_t row = last ? (int64_t)r : (int64_t)b * m + i;
#pragma unroll
            for (int j = 0; j < DPL; ++j) {
                const int64_t el = row * DI + lane * DPL + j;
                raw[i][j] = 0u;
                if (i < m)
                    raw[i][j] = p.tok_dtype == DT_F32 ? reinterpret_cast<const uint32_t*>(base)[el]
                                                      : (uint32_t)reinterpret_cast<const uint16_t*>(base)[el];
            }
        }
    }
};

// Logit of that entry, formed by one wave with compress_append's arithmetic,
// so its bits are those the pool will hold: the softmax weights of the
// group's logits by one wave, each dimension's products w_i x_i summed in
// token order, then the pool dtype's rounding; then scored from its stored
// value like the entries read from the pool (lane = head).  A row that is
// not the one new token of its sequence gets a NaN logit.
template <int KD, int NHT, int DI>
__device__ __forceinline__ void score_fresh(const IndexArgs& p, const FreshIn<DI>& in, int r, int b, int pos, int e,
                                            const uint8_t* q_lds, const float* w_lds, float* k_lds, float* out,
                                            uint32_t* lead) {
    constexpr int DPL = DI / 64;
    constexpr int QROWB = DI * 2 + 16;
    const int m = p.m, lane = threadIdx.x & 63;
    const bool ok = in.cu0 == r && in.cu1 == r + 1 && in.sp == pos;
    const float mx = wave_max(in.logit);
    const float ex = lane < m ? expf(in.logit - mx) : 0.0f;
    const float wsum = wave_sum(ex);
    const float w_mine = ex / wsum;
    float v[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) v[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i < m) {
            const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_mine), i));
#pragma unroll
            for (int j = 0; j < DPL; ++j) {
                const float x = p.tok_dtype == DT_F32 ? __uint_as_float(in.raw[i][j]) : bf16_to_f32(in.raw[i][j]);
                v[j] += fmaf(w, x, 0.0f);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < DPL; ++j) {
        float kd;
        if constexpr (KD == DT_FP8) kd = bf16_to_f32(fp8x8_to_bf16(f32_to_fp8(v[j]), 0u)[0] & 0xffffu);
        else kd = bf16_to_f32(f32_to_bf16(v[j]));
        k_lds[lane * DPL + j] = kd;
    }
    float l = 0.0f;
#pragma unroll
    for (int h0 = 0; h0 < NHT * 32; h0 += 64) {
        const int h = h0 + lane;
        if (h < NHT * 32) {
            const uint8_t* qh = q_lds + h * QROWB;
            float dot = 0.0f;
#pragma unroll 4
            for (int d = 0; d < DI; d += 8) {
                const u32x4 qq = *reinterpret_cast<const u32x4*>(qh + 2 * d);
                const f32x4 k0 = *reinterpret_cast<const f32x4*>(k_lds + d);
                const f32x4 k1 = *reinterpret_cast<const f32x4*>(k_lds + d + 4);
                dot = fmaf(bf16_to_f32(qq[0] & 0xffffu), k0[0], dot);
                dot = fmaf(bf16_to_f32(qq[0] >> 16), k0[1], dot);
                dot = fmaf(bf16_to_f32(qq[1] & 0xffffu), k0[2], dot);
                dot = fmaf(bf16_to_f32(qq[1] >> 16), k0[3], dot);
                dot = fmaf(bf16_to_f32(qq[2] & 0xffffu), k1[0], dot);
                dot = fmaf(bf16_to_f32(qq[2] >> 16), k1[1], dot);
                dot = fmaf(bf16_to_f32(qq[3] & 0xffffu), k1[2], dot);
                dot = fmaf(bf16_to_f32(qq[3] >> 16), k1[3], dot);
            }
            l = fmaf(w_lds[h], fmaxf(dot, 0.0f), l);
        }
    }
    l = wave_sum(l);
    if (lane == 0) {
        const float v_out = ok ? l : __builtin_nanf("");
        out[e] = v_out;
        if (lead) atomicAdd(&lead[order_key(v_out) >> (32 - kTopkLeadBits)], 1u);
    }
}

template <int KD, int NHT, int DI, bool Q8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd, kWavesPerSimd))) void
index_mfma_kernel(IndexArgs p) {
    constexpr int KS = DI / 16, HALF = DI / 2;
    constexpr int PF = key_depth<KD>();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 5, j = lane & 31;
    const int r_raw = (int)blockIdx.y;
    const bool row_ok = r_raw < p.num_rows;
    const int r = row_ok ? r_raw : p.num_rows - 1;
    const int tpw = p.tiles_per_wave;
    const int t_begin = ((int)blockIdx.x * 4 + wave) * tpw;
    const int b = checked(p.row_seq[r], 0, p.batch - 1, p.dbg, kDbgRow);
    const int pos = checked(p.row_pos[r], 0, p.max_pos, p.dbg, kDbgRow);
    const int n_all = visible_entries(pos, p.m);
    // the entry this row's token completes is scored by score_fresh
    const bool fresh = p.fresh && row_ok && (pos + 1) % p.m == 0;
    const int n = fresh ? n_all - 1 : n_all;
    // the wave whose tile range holds the fresh entry scores it after its
    // tiles; its inputs are requested now
    const bool fresh_owner = fresh && ((n_all - 1) >> 5) / p.tiles_per_wave == (int)blockIdx.x * 4 + wave;
    FreshIn<DI> fin;
    if (fresh_owner) fin.load(p, r, b);
    // The query (HI x DI bf16) and head weights of the workgroup's row are
    // staged in LDS once (rows padded by 16 bytes against bank conflicts);
    // every wave then reads its A operands from there instead of from L2.
    // They depend on the row index alone, so they are requested right after
    // the row's metadata: memory waits complete in issue order, so requested
    // after the first key tile they would wait for it.
    constexpr int QROWB = DI * 2 + 16;
    constexpr int UPR = DI * 2 / 16;                             // 16-byte units per head
    constexpr int QUNITS = NHT * 32 * UPR;
    constexpr int QU = (QUNITS + kThreads - 1) / kThreads;       // units per thread
    __shared__ __attribute__((aligned(16))) uint8_t q_lds[NHT * 32 * QROWB];
    __shared__ __attribute__((aligned(16))) float w_lds[NHT * 32];
    const uint8_t* qg = reinterpret_cast<const uint8_t*>(p.q) + (int64_t)r * p.HI * DI * 2;
    u32x4 qv[QU];
#pragma unroll
    for (int i = 0; i < QU; ++i) {
        const int u = min((int)threadIdx.x + kThreads * i, QUNITS - 1);      // branch-free, clamped
        qv[i] = *reinterpret_cast<const u32x4*>(qg + (int64_t)(u / UPR) * DI * 2 + (u % UPR) * 16);
    }
    const float wraw = p.w[(int64_t)r * p.HI + min((int)threadIdx.x, NHT * 32 - 1)];
    const int ntiles = (n + 31) >> 5;
    const int t_end = min(t_begin + tpw, ntiles);
    const bool work = row_ok && t_begin < t_end;
    const int sh = __builtin_ctz(256 / p.m);                    // E = 256/m entries per block, a power of two
    const int32_t* bt = p.block_table + (int64_t)b * p.max_blocks;
    const uint8_t* keys = reinterpret_cast<const uint8_t*>(p.keys);

    // Loads are issued unconditionally (tile indices clamped to the wave's
    // range) so the compiler's wait counts stay exact.  The block-table entry
    // of a tile is fetched one step ahead of its keys, the keys PF - 1 tiles
    // ahead of their MFMAs, in a ring of PF register sets addressed
    // statically (the tile loop is unrolled by PF).
    auto entry = [&](int tile) { return min(min(tile, t_end - 1) * 32 + j, n - 1); };
    auto table = [&](int tile) { return checked(bt[entry(tile) >> sh], 0, p.n_blocks - 1, p.dbg, kDbgBlock); };
    auto row = [&](int tile, int pb) -> int64_t {
        return ((int64_t)pb << sh) + (entry(tile) & ((1 << sh) - 1));
    };
    // Block-table entries of the first PF tiles, requested unconditionally
    // (entries clamped into the sequence's table row); then the query and
    // weights go to LDS, which waits for their loads only; then the first
    // key tiles are requested.
    int pbs[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i)
        pbs[i] = checked(bt[max(0, entry(t_begin + i)) >> sh], 0, p.n_blocks - 1, p.dbg, kDbgBlock);
#pragma unroll
    for (int i = 0; i < QU; ++i) {
        const int u = (int)threadIdx.x + kThreads * i;
        if (u < QUNITS) *reinterpret_cast<u32x4*>(&q_lds[(u / UPR) * QROWB + (u % UPR) * 16]) = qv[i];
    }
    if ((int)threadIdx.x < NHT * 32) w_lds[threadIdx.x] = wraw * p.s_I;
    // leading-digit counts of this workgroup's logits (fused decode launch),
    // added to the row's counts in memory at the end
    constexpr int kLeadBins = 1 << kTopkLeadBits;
    __shared__ __attribute__((aligned(16))) uint32_t lead_lds[kLeadBins];
    uint32_t* const lead = p.lead_hist ? lead_lds : nullptr;
    if (lead)
        for (int i = (int)threadIdx.x; i < kLeadBins / 4; i += kThreads)
            reinterpret_cast<u32x4*>(lead_lds)[i] = u32x4{0u, 0u, 0u, 0u};
    int pb_next = pbs[PF - 1];
    RawKey<KD, KS> kr[PF];
    if (work) {
#pragma unroll
        for (int i = 0; i < PF - 1; ++i) load_key<KD, KS>(keys, row(t_begin + i, pbs[i]), g, kr[i]);
    }
    __syncthreads();
    // FP8 queries: quantised in place (the fresh entry's score below reads
    // the same values), their FP8 codes as A operands of the FP8 MFMA, head
    // 32t + j, k-block s8 = dims [g*HALF + 32 s8, +32), with the head's
    // exponent as the operand's E8M0 scale
    constexpr int KS8 = HALF / 32;
    constexpr int Q8ROWB = DI + 16;                              // code rows padded against bank conflicts
    __shared__ int x_lds[NHT * 32];
    __shared__ __attribute__((aligned(16))) uint8_t q8_lds[Q8 ? NHT * 32 * Q8ROWB : 16];
    i32x8 qa8[Q8 ? NHT : 1][Q8 ? KS8 : 1];
    int sa[NHT];
    if constexpr (Q8) {
        quantize_query_lds<NHT, DI, QROWB, Q8ROWB>(q_lds, q8_lds, x_lds);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < NHT; ++t) {
            sa[t] = x_lds[32 * t + j] + 127;
#pragma unroll
            for (int s8 = 0; s8 < KS8; ++s8) {
                const uint8_t* src = &q8_lds[(32 * t + j) * Q8ROWB + g * HALF + 32 * s8];
                const u32x4 lo = *reinterpret_cast<const u32x4*>(src), hi = *reinterpret_cast<const u32x4*>(src + 16);
                qa8[t][s8] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
        }
    }
    // bf16 queries as A operands: head 32t + j, dims [g*HALF + 8s, +8)
    bf16x8 qa[Q8 ? 1 : NHT][Q8 ? 1 : KS];
    if constexpr (!Q8) {
#pragma unroll
        for (int t = 0; t < NHT; ++t)
#pragma unroll
            for (int s = 0; s < KS; ++s)
                qa[t][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                          &q_lds[(32 * t + j) * QROWB + (g * HALF + 8 * s) * 2]));
    }
    // head weights are read from LDS per tile, in C-layout order: head
    // 32t + 8(v/4) + 4g + v%4, four consecutive heads per 16-byte read
    const float* wrow = &w_lds[4 * g];

    float* out = p.logits + (int64_t)r * p.ld;
    auto step = [&](auto J, int tile) __attribute__((always_inline)) {
        constexpr int cur = decltype(J)::value, ld = (cur + PF - 1) % PF;
        RawKey<KD, KS>& kc = kr[cur];
        const int pb2 = table(tile + PF);
        load_key<KD, KS>(keys, row(tile + PF - 1, pb_next), g, kr[ld]);
        pb_next = pb2;
        f32x16 acc[NHT];
#pragma unroll
        for (int t = 0; t < NHT; ++t) acc[t] = f32x16{};
        if constexpr (Q8) {
#pragma unroll
            for (int s8 = 0; s8 < KS8; ++s8) {
                const i32x8 kb = key_operand8<KS>(kc, s8);
#pragma unroll
                for (int t = 0; t < NHT; ++t)
                    acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa8[t][s8], kb, acc[t], 0, 0, 0, sa[t], 0,
                                                                            127);
            }
        } else {
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int t = 0; t < NHT; ++t)
                    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[t][s], key_operand<KD, KS>(kc, s), acc[t], 0, 0,
                                                                    0);
        }
        float l = 0.0f;
#pragma unroll
        for (int t = 0; t < NHT; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 w4 = *reinterpret_cast<const f32x4*>(wrow + 32 * t + 8 * q);
#pragma unroll
                for (int i = 0; i < 4; ++i) l = fmaf(w4[i], fmaxf(acc[t][4 * q + i], 0.0f), l);
            }
        l = sum_halves(l);
        const int e = tile * 32 + j;
        if (g == 0 && e < n) {
            out[e] = l;
            if (lead) atomicAdd(&lead_lds[order_key(l) >> (32 - kTopkLeadBits)], 1u);
        }
    };
    if (work)
        for (int tile = t_begin; tile < t_end; tile += PF) unroll_steps<0, PF>(step, tile, t_end);
    if (fresh_owner) {
        __shared__ __attribute__((aligned(16))) float fresh_k[DI];
        score_fresh<KD, NHT, DI>(p, fin, r, b, pos, n_all - 1, q_lds, w_lds, fresh_k, out, lead);
    }
    if (lead) {
        __syncthreads();
        uint32_t* const row_lead = p.lead_hist + (int64_t)r * kLeadBins;
        for (int i = (int)threadIdx.x; i < kLeadBins / 4; i += kThreads) {
            const u32x4 c = reinterpret_cast<const u32x4*>(lead_lds)[i];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (c[q]) atomicAdd(&row_lead[4 * i + q], c[q]);
        }
    }
}

// Many rows (prefill): a workgroup of eight waves covers 8 RPW rows, RPW
// per wave, and a range of tiles.  Rows of one sequence read the same keys,
// so each 32-entry key tile is staged in LDS once (rows padded by 16 bytes, a
// ring of three stages, the raw bytes of the next two tiles in flight in
// registers) and every wave takes its B operands from there, once per tile
// for all of its rows; the queries stay in VGPRs as A operands.  One barrier
// per tile: the stage written in step t was last read in step t - 2, before
// the barrier of step t - 1.  Rows of a workgroup that belong to different
// sequences are handled one sequence after another, the other rows' waves
// only helping to stage keys.
constexpr int kRowWaves = 8;
constexpr int kRowThreads = kRowWaves * 64;
constexpr int kRowStages = 3;
// Rows per wave: two, so each B operand read from LDS feeds both rows'
// MFMAs and a tile's barrier covers twice the work (prefill_8k indexer 4.70
// -> 4.26 ms, 40 % of the bf16 MFMA peak); one where the tile's B operands
// alone take 64 registers (d_I = 256), as two rows' queries would then spill.
template <int DI>
constexpr int rows_per_wave() {
    return DI / 16 <= 8 ? 2 : 1;
}

template <int KD, int NHT, int DI, int RPW>
__global__ __launch_bounds__(kRowThreads) void index_rows_kernel(IndexArgs p) {
    constexpr int KS = DI / 16, HALF = DI / 2;
    constexpr int KB = KD == DT_BF16 ? DI * 2 : DI;               // bytes of one key
    constexpr int KBP = KB + 16;                                   // padded LDS row
    constexpr int UPK = KB / 16;                                   // 16-byte units per key
    constexpr int UPT = (32 * UPK + kRowThreads - 1) / kRowThreads;   // units per thread per tile
    constexpr int NR = kRowWaves * RPW;                            // rows per workgroup
    __shared__ __attribute__((aligned(16))) uint8_t kst[kRowStages][32 * KBP];
    __shared__ __attribute__((aligned(16))) float w_lds[NR][NHT * 32];
    __shared__ int seq_lds[NR], n_lds[NR];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, j = lane & 31;
    // this wave's rows: slots RPW wave + q
    bool row_ok[RPW];
    int rr[RPW], b[RPW], n[RPW];
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
        const int r = (int)blockIdx.y * NR + wave * RPW + q;
        row_ok[q] = r < p.num_rows;
        rr[q] = row_ok[q] ? r : p.num_rows - 1;
        b[q] = checked(p.row_seq[rr[q]], 0, p.batch - 1, p.dbg, kDbgRow);
        n[q] = row_ok[q] ? visible_entries(checked(p.row_pos[rr[q]], 0, p.max_pos, p.dbg, kDbgRow), p.m) : 0;
    }
    const int tpb = p.tiles_per_wave;
    const int t_begin = (int)blockIdx.x * tpb;
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
        if (lane == 0) { seq_lds[wave * RPW + q] = b[q]; n_lds[wave * RPW + q] = n[q]; }
        for (int h = lane; h < NHT * 32; h += 64) w_lds[wave * RPW + q][h] = p.w[(int64_t)rr[q] * p.HI + h] * p.s_I;
    }
    // queries as A operands: row q, head 32t + j, dims [g*HALF + 8s, +8)
    bf16x8 qa[RPW][NHT][KS];
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
        const uint8_t* qg = reinterpret_cast<const uint8_t*>(p.q) + (int64_t)rr[q] * p.HI * DI * 2;
#pragma unroll
        for (int t = 0; t < NHT; ++t)
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2)
                qa[q][t][s2] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(qg + ((int64_t)(32 * t + j) * DI + g * HALF + 8 * s2) * 2));
    }
    __syncthreads();
    const int sh = __builtin_ctz(256 / p.m);
    const uint8_t* keys = reinterpret_cast<const uint8_t*>(p.keys);

    for (int i = 0; i < NR; ++i) {
        const int sb = seq_lds[i];
        bool first = true;
        int nmax = 0;
        for (int k = 0; k < NR; ++k) {
            if (seq_lds[k] == sb) {
                if (k < i) first = false;
                nmax = max(nmax, n_lds[k]);
            }
        }
        if (!first) continue;
        const int t_end = min(t_begin + tpb, (nmax + 31) >> 5);
        if (t_begin >= t_end) continue;
        bool mine[RPW], any = false;
#pragma unroll
        for (int q = 0; q < RPW; ++q) {
            mine[q] = row_ok[q] && b[q] == sb;
            any = any || mine[q];
        }
        const int32_t* bt = p.block_table + (int64_t)sb * p.max_blocks;
        // this thread's units of a tile: key u / UPK, part u % UPK, u = tid + kRowThreads * i
        auto load = [&](int tile, u32x4 (&v)[UPT]) __attribute__((always_inline)) {
#pragma unroll
            for (int q = 0; q < UPT; ++q) {
                const int u = min(tid + kRowThreads * q, 32 * UPK - 1);
                const int e = min(min(tile, t_end - 1) * 32 + u / UPK, nmax - 1);
                const int64_t row =
                    ((int64_t)checked(bt[e >> sh], 0, p.n_blocks - 1, p.dbg, kDbgBlock) << sh) + (e & ((1 << sh) - 1));
                v[q] = *reinterpret_cast<const u32x4*>(keys + row * KB + (u % UPK) * 16);
            }
        };
        auto store = [&](int stage, const u32x4 (&v)[UPT]) __attribute__((always_inline)) {
#pragma unroll
            for (int q = 0; q < UPT; ++q) {
                const int u = tid + kRowThreads * q;
                if (u < 32 * UPK) *reinterpret_cast<u32x4*>(&kst[stage][(u / UPK) * KBP + (u % UPK) * 16]) = v[q];
            }
        };
        u32x4 ra[UPT], rb[UPT];
        load(t_begin, ra);
        load(t_begin + 1, rb);
        store(0, ra);
        load(t_begin + 2, ra);
        __syncthreads();
        auto step = [&](int tile, int stage, u32x4 (&nxt)[UPT]) __attribute__((always_inline)) {
            // registers `nxt` hold tile + 1: into the next stage, then refill with tile + 3
            if (tile + 1 < t_end) store(stage == kRowStages - 1 ? 0 : stage + 1, nxt);
            load(tile + 3, nxt);
            if (any) {
                // the tile's B operands, read once for the wave's rows
                const uint8_t* kb = &kst[stage][j * KBP];
                bf16x8 kop[KS];
#pragma unroll
                for (int s2 = 0; s2 < KS; ++s2) {
                    if constexpr (KD == DT_BF16) {
                        kop[s2] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kb + (g * HALF + 8 * s2) * 2));
                    } else {
                        const u32x2 c = *reinterpret_cast<const u32x2*>(kb + g * HALF + 8 * s2);
                        kop[s2] = __builtin_bit_cast(bf16x8, fp8x8_to_bf16(c[0], c[1]));
                    }
                }
                const int e = tile * 32 + j;
#pragma unroll
                for (int q = 0; q < RPW; ++q) {
                    if (!mine[q]) continue;
                    f32x16 acc[NHT];
#pragma unroll
                    for (int t = 0; t < NHT; ++t) acc[t] = f32x16{};
#pragma unroll
                    for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
                        for (int t = 0; t < NHT; ++t)
                            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[q][t][s2], kop[s2], acc[t], 0, 0, 0);
                    const float* wrow = &w_lds[wave * RPW + q][4 * g];
                    float l = 0.0f;
#pragma unroll
                    for (int t = 0; t < NHT; ++t)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const f32x4 w4 = *reinterpret_cast<const f32x4*>(wrow + 32 * t + 8 * v);
#pragma unroll
                            for (int i4 = 0; i4 < 4; ++i4) l = fmaf(w4[i4], fmaxf(acc[t][4 * v + i4], 0.0f), l);
                        }
                    l = sum_halves(l);
                    if (g == 0 && e < n[q]) p.logits[(int64_t)rr[q] * p.ld + e] = l;
                }
            }
            __syncthreads();
        };
        int stage = 0;
        for (int tile = t_begin; tile < t_end; tile += 2) {
            step(tile, stage, rb);
            stage = stage == kRowStages - 1 ? 0 : stage + 1;
            if (tile + 1 < t_end) {
                step(tile + 1, stage, ra);
                stage = stage == kRowStages - 1 ? 0 : stage + 1;
            }
        }
    }
}

// fp32 path (tiny workloads): one thread per (row, entry), plain FMAs.
__global__ __launch_bounds__(kThreads) void index_f32_kernel(IndexArgs p) {
    const int r = blockIdx.y;
    const int e = blockIdx.x * kThreads + threadIdx.x;
    const int n = visible_entries(checked(p.row_pos[r], 0, p.max_pos, p.dbg, kDbgRow), p.m);
    if (e >= n) return;
    const int E = 256 / p.m;
    const int b = checked(p.row_seq[r], 0, p.batch - 1, p.dbg, kDbgRow);
    const int64_t row =
        (int64_t)checked(p.block_table[(int64_t)b * p.max_blocks + e / E], 0, p.n_blocks - 1, p.dbg, kDbgBlock) * E +
        e % E;
    const float* k = reinterpret_cast<const float*>(p.keys) + row * p.dI;
    const float* q = reinterpret_cast<const float*>(p.q) + (int64_t)r * p.HI * p.dI;
    float l = 0.0f;
    for (int h = 0; h < p.HI; ++h) {
        float dot = 0.0f;
        for (int d = 0; d < p.dI; ++d) dot = fmaf(q[h * p.dI + d], k[d], dot);
        l = fmaf(p.w[(int64_t)r * p.HI + h], fmaxf(dot, 0.0f), l);
    }
    p.logits[(int64_t)r * p.ld + e] = p.s_I * l;
}

template <int KD, int NHT, int DI>
hipError_t launch_mfma(IndexArgs a, int max_entries, hipStream_t stream) {
    const int max_tiles = (max_entries + 31) / 32;
    if (a.num_rows >= 64) {
        constexpr int kTilesPerGroup = 64;
        a.tiles_per_wave = kTilesPerGroup;
        constexpr int RPW = rows_per_wave<DI>();
        dim3 grid((max_tiles + kTilesPerGroup - 1) / kTilesPerGroup,
                  (a.num_rows + kRowWaves * RPW - 1) / (kRowWaves * RPW));
        hipLaunchKernelGGL((index_rows_kernel<KD, NHT, DI, RPW>), grid, dim3(kRowThreads), 0, stream, a);
    } else {
        // one round of waves over the GPU (256 CUs x 4 SIMDs x waves per
        // SIMD), each streaming a contiguous tile range
        const int64_t waves = 256 * 4 * kWavesPerSimd;
        const int64_t wave_tiles = (int64_t)a.num_rows * max_tiles;
        int tpw = (int)((wave_tiles + waves - 1) / waves);
        if (tpw < 1) tpw = 1;
        a.tiles_per_wave = tpw;
        dim3 grid((max_tiles + 4 * tpw - 1) / (4 * tpw), a.num_rows);
        if constexpr (KD == DT_FP8) {
            if (a.q8) {
                hipLaunchKernelGGL((index_mfma_kernel<KD, NHT, DI, true>), grid, dim3(kThreads), 0, stream, a);
                return hipGetLastError();
            }
        }
        hipLaunchKernelGGL((index_mfma_kernel<KD, NHT, DI, false>), grid, dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

bool index_supported(int q_dtype, int key_dtype, int HI, int dI) {
    if (q_dtype == DT_F32) return key_dtype == DT_F32 && HI >= 1 && dI >= 1;
    if (q_dtype != DT_BF16 || (key_dtype != DT_BF16 && key_dtype != DT_FP8)) return false;
    // the query stays in VGPRs: (HI/32) * (dI/16) <= 16 operand registers of 8 bf16
    return (HI == 32 || HI == 64 || HI == 128) && (dI == 64 || dI == 128 || dI == 256) && (HI / 32) * (dI / 16) <= 16;
}

hipError_t launch_index_logits(const IndexArgs& a, int max_entries, hipStream_t stream) {
    if (a.num_rows <= 0 || max_entries <= 0) return hipSuccess;
    const int qdt = a.key_dtype == DT_F32 ? DT_F32 : DT_BF16;
    if (qdt == DT_F32) {
        dim3 grid((max_entries + kThreads - 1) / kThreads, a.num_rows);
        hipLaunchKernelGGL(index_f32_kernel, grid, dim3(kThreads), 0, stream, a);
        return hipGetLastError();
    }
#define LCCA_IDX_CASE(KD, NHT, DI) \
    if (a.key_dtype == KD && a.HI == 32 * NHT && a.dI == DI) return launch_mfma<KD, NHT, DI>(a, max_entries, stream);
#define LCCA_IDX_DT(KD) LCCA_IDX_CASE(KD, 1, 64) LCCA_IDX_CASE(KD, 1, 128) LCCA_IDX_CASE(KD, 1, 256) \
    LCCA_IDX_CASE(KD, 2, 64) LCCA_IDX_CASE(KD, 2, 128) LCCA_IDX_CASE(KD, 4, 64)
    LCCA_IDX_DT(DT_BF16) LCCA_IDX_DT(DT_FP8)
#undef LCCA_IDX_DT
#undef LCCA_IDX_CASE
    return hipErrorInvalidValue;
}

}  // namespace lcca
