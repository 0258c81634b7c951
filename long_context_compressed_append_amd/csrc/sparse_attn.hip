// sparse_attn_fwd: single-KV-head attention of H query heads over the
// selected compressed entries plus the sliding window, one joint softmax.
//
// [Page "vLLM uveo DeepSeek V4 s 8,7x manjim KV cacheom", section "Kako
//  funkcionira optimizacija KV cachea?": shared KV vectors (one vector is key
//  and value), attention restricted to the top-k compressed tokens, and a
//  local window of full vectors for recent context.  Page "DeepSeek-V4.1-Flash
//  ve vLLM: kde se vzala 5,3x vyssi propustnost", section "Vykon neprinesl
//  jeden kernel": the fused attention reads a 4-bit compressed cache; here
//  MXFP4 (OCP) or bf16 entries and an FP8 or bf16 window are upconverted
//  exactly to bf16 on their way into LDS.]
//
// Key list of a row: the selected entries (topk slots, or every visible
// entry), padded with masked slots to a multiple of 32, then the window
// tokens.  So every 32-key tile holds either pool entries or window tokens.
//
// bf16/MFMA path.  A workgroup = (row, range of tiles, group of 64 heads)
// with eight waves: two groups of 32 heads, each over four quarters of the
// shared-KV dimension.  Pipeline per workgroup:
//   prologue: the block-table range and the top-k indices the split needs are
//     copied to LDS, so resolving a key to its storage row is two LDS reads;
//   loads:    each tile's raw bytes (bf16, FP8 or MXFP4 + E8M0 scales) are
//     loaded into registers P tiles ahead of their use (static register sets,
//     loop unrolled by P), converted exactly to bf16 and written to one of two
//     padded LDS stages; two barriers per tile;
//   compute:  partial S^T = K Q^T over a quarter of D with MFMA 16x16x32
//     (A = keys from LDS, B = the wave's queries, resident in VGPRs), summed
//     through LDS by the wave that owns eight of the group's heads; online
//     softmax in the exp2 domain; O^T += V^T P^T over a quarter of the value
//     dims with V^T read from the same LDS tile by ds_read_b64_tr_b16
//     (K = V); P enters as bf16 hi + lo so the value weights keep 16
//     significant bits; FP8 window scales multiply the scores and are folded
//     into P.
// Keys are split across workgroups when the rows alone cannot fill the GPU;
// the partial (max, sum, O) states go to the workspace and a merge kernel
// (one workgroup per row and head) combines them.  For fp32 outputs O stays
// fp32; for bf16 outputs O / sum is stored as fp16 (11 significant bits,
// eight times finer than the output's rounding) with a power-of-two range
// scale per split, head and quarter of the value dims.
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace lcca {

namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kKeys = 32;              // keys per tile

// LDS-typed pointers: stage addresses are formed in address space 3 so no
// generic-to-LDS conversion is ever needed on a run-time selected pointer.
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) int32_t lds_i32;

template <int N>
struct IntC {
    static constexpr int value = N;
};

template <int D>
struct Geo {
    static constexpr int ROWB = D * 2 + 32;          // padded bf16 row (bank-conflict counters: 0.37 conflict
                                                     // cycles per LDS-active cycle against 1.0 with 16 B)
    static constexpr int STAGE = kKeys * ROWB;
    static constexpr int U16 = D / 8;                // 16-B bf16 units per key
};

// Row-level key geometry.
struct RowKeys {
    int b, p, n;          // sequence, position, visible entries
    int nsel;             // selected (or visible) entries in the list
    int sel_tiles;        // tiles of the selected part (padded to 32)
    int t0, nwin;         // first window position, window tokens
    int tiles;            // total tiles of the row
};

__device__ inline RowKeys row_keys(const AttnArgs& a, int r) {
    RowKeys k;
    k.b = a.row_seq[r];
    k.p = a.row_pos[r];
    k.n = visible_entries(k.p, a.m);
    k.nsel = a.topk ? a.k : k.n;
    k.sel_tiles = (k.nsel + kKeys - 1) / kKeys;
    k.t0 = max(0, k.p - a.window + 1);
    k.nwin = k.p - k.t0 + 1;
    k.tiles = k.sel_tiles + (k.nwin + kKeys - 1) / kKeys;
    return k;
}

// Storage row of slot j of the selected part (-1: masked).  The block-table
// range of the split is in LDS.
__device__ __forceinline__ int64_t pool_row(const AttnArgs& a, const RowKeys& rk, int j, const lds_i32* idx_lds, int idx0,
                                            const lds_i32* bt_lds, int blk0) {
    const int g = a.topk ? idx_lds[j - idx0] : j;
    const bool ok = j < rk.nsel && g >= 0 && g < rk.n;
    const int sh = __builtin_ctz(256 / a.m);                  // E = 256/m entries per block, a power of two
    const int gc = ok ? g : blk0 << sh;
    const int lb = gc >> sh;
    const int pb = bt_lds[lb - blk0];
    return ok ? ((int64_t)pb << sh) + (gc & ((1 << sh) - 1)) : -1;
}

// Tile staging.  NT / 32 threads share a key: thread t stages key t / (NT/32)
// of the 32 keys of a tile, 16-byte parts (t % (NT/32)) + (NT/32) i, so each
// thread resolves one storage row per tile and its loads and LDS writes
// differ only by immediate offsets.  Raw bytes are loaded into registers
// ahead of use and converted exactly to bf16 when they are written to LDS;
// loaded values are consumed only then, so the loads stay in flight.
template <int NU>
struct TileRegs {
    u32x4 v[NU];
    uint32_t sc[NU];      // E8M0 scale of each MXFP4 part
    float kscale;         // FP8 window scale of this thread's key (1 otherwise)
    bool valid;           // this thread's key is not masked
};

template <int KVD, int WD, int D, int NT>
struct Tiler {
    static constexpr int kThreadsPerKey = NT / kKeys;
    static_assert(NT % kKeys == 0, "whole keys per workgroup");
    // 16-byte source parts per key: bf16 rows, FP8 rows, MXFP4 rows
    static constexpr int UB = D / 8, UF8 = D / 16, UF4 = D / 32;
    static constexpr int UPK_W = WD == DT_BF16 ? UB : UF8;
    static constexpr int UPK_P = KVD == DT_BF16 ? UB : UF4;
    static constexpr int NU_W = (UPK_W + kThreadsPerKey - 1) / kThreadsPerKey;
    static constexpr int NU_P = (UPK_P + kThreadsPerKey - 1) / kThreadsPerKey;
    static constexpr int NU = NU_W > NU_P ? NU_W : NU_P;

    // Where this thread's key of tile `tile` (row-local tile index) is
    // stored.  `live` false (a tile past the split): row 0 is read and
    // nothing is used; issuing those loads anyway keeps the number of loads
    // per step fixed, so the compiler's wait counts stay exact.  Masked keys
    // also read row 0 and are zeroed when stored.
    struct Src {
        int64_t row;
        bool ok, win;
    };
    __device__ __forceinline__ static Src resolve(const AttnArgs& a, const RowKeys& rk, int tile, bool live,
                                                  const lds_i32* idx_lds, int idx0, const lds_i32* bt_lds, int blk0) {
        const int key = (int)threadIdx.x / kThreadsPerKey;
        Src s;
        s.win = live && tile >= rk.sel_tiles;                       // uniform over the workgroup
        if (s.win) {
            const int w = (tile - rk.sel_tiles) * kKeys + key;
            s.ok = w < rk.nwin;
            s.row = (int64_t)rk.b * a.win_cap + (rk.t0 + (s.ok ? w : 0)) % a.win_cap;
        } else {
            const int64_t prow = pool_row(a, rk, (live ? tile * kKeys : idx0) + key, idx_lds, idx0, bt_lds, blk0);
            s.ok = live && prow >= 0;
            s.row = s.ok ? prow : 0;
        }
        return s;
    }

    // Issue the loads of a resolved key into registers.  One load sequence
    // serves both sources (the row's address and part count are selected,
    // parts past the row re-read part 0): a register written on two branch
    // paths would make the compiler wait at the join for every older load
    // still in flight.
    __device__ __forceinline__ static void issue(const AttnArgs& a, const Src& s, TileRegs<NU>& R) {
        const int sub = (int)threadIdx.x % kThreadsPerKey;
        constexpr int64_t WROWB = WD == DT_BF16 ? 2 * D : D;
        constexpr int64_t PROWB = KVD == DT_BF16 ? 2 * D : D / 2;
        const uint8_t* base = reinterpret_cast<const uint8_t*>(s.win ? a.win_data : a.kv_data);
        const uint8_t* src = base + s.row * (s.win ? WROWB : PROWB);
        const int upk = s.win ? UPK_W : UPK_P;
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int part = sub + kThreadsPerKey * i;
            const int pc = part < upk ? part : 0;
            R.v[i] = *reinterpret_cast<const u32x4*>(src + pc * 16);
            if constexpr (KVD == DT_MXFP4) {
                // E8M0 scales of the pool row (row 0's for window tiles, unused)
                const int ps = part < UPK_P ? part : 0;
                const uint32_t e = reinterpret_cast<const uint8_t*>(a.kv_scale)[(s.win ? 0 : s.row) * (D / 32) + ps];
                R.sc[i] = s.win ? 127u : e;
            } else {
                R.sc[i] = 127u;
            }
        }
        if constexpr (WD == DT_FP8) {
            const float ws = a.win_scale[s.win ? s.row : 0];
            R.kscale = s.win ? ws : 1.0f;
        } else {
            R.kscale = 1.0f;
        }
        R.valid = s.ok;
    }

    // Convert the registers of tile `tile` to bf16 and write them to an LDS
    // stage.  kmeta[key]: the key's value scale (FP8 window scale, 1, or -1
    // for a masked key), which also multiplies its score.
    __device__ __forceinline__ static void store(const RowKeys& rk, int tile, const TileRegs<NU>& R, lds_u8* stage,
                                                 lds_f32* kmeta) {
        const int tid = threadIdx.x;
        const int key = tid / kThreadsPerKey, sub = tid % kThreadsPerKey;
        if (sub == 0) kmeta[key] = R.valid ? R.kscale : -1.0f;
        lds_u8* dst = stage + key * Geo<D>::ROWB;
        if (tile >= rk.sel_tiles) store_parts<WD, UPK_W, NU_W>(R, dst, sub);
        else store_parts<KVD, UPK_P, NU_P>(R, dst, sub);
    }

    template <int SRC, int UPK, int NUS>
    __device__ __forceinline__ static void store_parts(const TileRegs<NU>& R, lds_u8* dst, int sub) {
        const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < NUS; ++i) {
            const int part = sub + kThreadsPerKey * i;
            const bool in = (i + 1) * kThreadsPerKey <= UPK || part < UPK;
            const u32x4 v = R.valid ? R.v[i] : zero;
            if (SRC == DT_BF16) {
                if (in) *reinterpret_cast<lds_u32x4*>(dst + part * 16) = v;
            } else if (SRC == DT_FP8) {
                // 16 E4M3 codes -> 16 bf16 (exact)
                const u32x4 o0 = fp8x8_to_bf16(v[0], v[1]);
                const u32x4 o1 = fp8x8_to_bf16(v[2], v[3]);
                if (in) {
                    *reinterpret_cast<lds_u32x4*>(dst + part * 32) = o0;
                    *reinterpret_cast<lds_u32x4*>(dst + part * 32 + 16) = o1;
                }
            } else {
                // 32 E2M1 codes with one E8M0 scale -> 32 bf16 (exact)
                const int X = R.valid ? (int)R.sc[i] - 127 : 0;
                const u32x4 o0 = fp4x8_to_bf16(v[0], X), o1 = fp4x8_to_bf16(v[1], X);
                const u32x4 o2 = fp4x8_to_bf16(v[2], X), o3 = fp4x8_to_bf16(v[3], X);
                if (in) {
                    *reinterpret_cast<lds_u32x4*>(dst + part * 64) = o0;
                    *reinterpret_cast<lds_u32x4*>(dst + part * 64 + 16) = o1;
                    *reinterpret_cast<lds_u32x4*>(dst + part * 64 + 32) = o2;
                    *reinterpret_cast<lds_u32x4*>(dst + part * 64 + 48) = o3;
                }
            }
        }
    }
};

// Per-wave tile computation.  The eight waves of a workgroup form two head
// groups of 32 heads, each split into four quarters of the shared-KV
// dimension: a wave holds its head group's queries over its quarter of D in
// VGPRs and the O^T accumulators of its quarter of the value dims for all 32
// heads, so every key fragment read from LDS feeds 32 heads.  Per tile:
//   scores:  partial S^T = K Q^T over the wave's quarter of D (MFMA 16x16x32,
//            keys on M), written to the wave's slot of the exchange buffer;
//   softmax: (after a barrier) wave q of a head group owns heads 8q .. 8q+7:
//            it sums the four partials of its heads, runs the online softmax
//            (lane: one head, four keys; the tile max over eight lanes),
//            and writes P as bf16 hi + lo and the heads' rescale factors;
//   P V:     (after a barrier) every wave rescales its accumulators where a
//            head's reference max moved and adds V^T P^T over its value
//            quarter, V^T read from the same LDS tile by ds_read_b64_tr_b16.
template <int D, int DV>
struct QuarterWave {
    static constexpr int KS_ALL = D / 32;                   // k-steps of S^T over D
    static constexpr int KSQ = (KS_ALL + 3) / 4;            // most k-steps of one quarter
    static constexpr int DVQ = DV / 4;                       // value dims per quarter
    static constexpr int NDQ = DVQ / 16;                     // 16-dim tiles of O^T per wave
    static_assert(D % 32 == 0 && DV % 64 == 0, "shape");
    static constexpr int XROW = kKeys * 4 + 16;              // exchange row: 32 fp32 scores of a head, padded
    static constexpr int XSLOT = 32 * XROW;                  // one wave's partial S^T (32 heads)
    static constexpr int PROW = kKeys * 2 + 16;              // P row: 32 bf16 weights of a head, padded
    static constexpr int PGRP = 32 * PROW;                   // one head group's P (hi or lo)
    bf16x8 qb[2][KSQ];
    f32x4 o[2][NDQ];
    float m_run, l_run;            // owner state of head 8q + (lane & 7)
    int ks0, ksn;                  // this quarter's k-steps

    __device__ __forceinline__ void init(const AttnArgs& a, int r, int head0, int g, int c16, int q) {
        constexpr int base = KS_ALL / 4, extra = KS_ALL % 4;
        ks0 = q * base + min(q, extra);
        ksn = base + (q < extra ? 1 : 0);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const uint16_t* qp =
                reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)r * a.H + head0 + 16 * hb + c16) * D + ks0 * 32 + 8 * g;
#pragma unroll
            for (int s = 0; s < KSQ; ++s)
                qb[hb][s] = s < ksn ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 32 * s))
                                    : bf16x8{};
#pragma unroll
            for (int dt = 0; dt < NDQ; ++dt) o[hb][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        m_run = -INFINITY;
        l_run = 0.0f;
    }

    // Partial S^T of the tile over this quarter of D, into the wave's exchange
    // slot as [head][key] rows.
    __device__ __forceinline__ void scores(const lds_u8* lds, lds_u8* xs_mine, int g, int c16) const {
        constexpr int ROWB = Geo<D>::ROWB;
        f32x4 sacc[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) sacc[kt][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const lds_u8* kbase = lds + c16 * ROWB + (ks0 * 32 + 8 * g) * 2;
#pragma unroll
        for (int s = 0; s < KSQ; ++s) {
            if (s < ksn) {
                bf16x8 kA[2];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
                    kA[kt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const lds_u32x4*>(kbase + kt * 16 * ROWB + 64 * s));
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int hb = 0; hb < 2; ++hb)
                        sacc[kt][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA[kt], qb[hb][s], sacc[kt][hb], 0, 0, 0);
            }
        }
        // lane: keys kt*16 + 4g .. +3 of head hb*16 + c16
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                *reinterpret_cast<lds_f32x4*>(xs_mine + (hb * 16 + c16) * XROW + (kt * 16 + 4 * g) * 4) = sacc[kt][hb];
    }

    // Owner softmax of heads 8q .. 8q+7 of the head group: lane (h8 = lane & 7,
    // kg = lane >> 3) takes keys 4kg .. 4kg+3 of head 8q + h8.  xs_grp: the
    // head group's four exchange slots; kmeta: each key's value scale (FP8
    // window scale, 1, or -1 for a masked key).  Writes P hi/lo in the order
    // the P V operands read it and the head's rescale factor alpha.
    __device__ __forceinline__ void softmax(const lds_u8* xs_grp, const lds_f32* kmeta, lds_u8* p_hi, lds_u8* p_lo,
                                            lds_f32* alpha, int lane, int q, float scale_log2) {
        const int h8 = lane & 7, kg = lane >> 3, hq = 8 * q + h8;
        f32x4 s = *reinterpret_cast<const lds_f32x4*>(xs_grp + hq * XROW + 16 * kg);
#pragma unroll
        for (int src = 1; src < 4; ++src)
            s += *reinterpret_cast<const lds_f32x4*>(xs_grp + src * XSLOT + hq * XROW + 16 * kg);
        const f32x4 km = *reinterpret_cast<const lds_f32x4*>(kmeta + 4 * kg);
        float x[4];
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            x[v] = km[v] >= 0.0f ? s[v] * (scale_log2 * km[v]) : -INFINITY;
            mx = fmaxf(mx, x[v]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 8));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // Lazy rescaling: the reference max m_run moves only when the tile's
        // max exceeds it by more than 8 (log2 units), so most tiles leave the
        // accumulators untouched; weights relative to m_run stay <= 2^8.
        float al = 1.0f;
        if (mx > m_run + 8.0f) {
            al = exp2f(m_run - mx);      // 0 while m_run = -inf
            l_run *= al;
            m_run = mx;
        }
        // reference for the exponent: m_run, or 0 while every key so far is
        // masked (then every x is -inf and every p is 0)
        const float mref = m_run == -INFINITY ? 0.0f : m_run;
        float w[4], psum = 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            // x - mref <= 8: v_exp_f32 directly (results below 2^-126 may
            // flush to zero, far below the sum's precision)
            const float p = __builtin_amdgcn_exp2f(x[v] - mref);
            psum += p;
            w[v] = p * km[v];            // masked keys: p = 0; FP8 window keys carry their scale
        }
        l_run += psum;
        const uint32_t h0 = cvt_pk_bf16(w[0], w[1]), h1 = cvt_pk_bf16(w[2], w[3]);
        const uint32_t l0 = cvt_pk_bf16(w[0] - __uint_as_float(h0 << 16), w[1] - __uint_as_float(h0 & 0xffff0000u));
        const uint32_t l1 = cvt_pk_bf16(w[2] - __uint_as_float(h1 << 16), w[3] - __uint_as_float(h1 & 0xffff0000u));
        // P row order: keys 0-3, 16-19, 4-7, 20-23, ... so that operand lane
        // group g reads keys 4g .. 4g+3 and 16+4g .. 16+4g+3 as one 16-byte run
        const int off = hq * PROW + (kg < 4 ? 16 * kg : 16 * (kg - 4) + 8);
        *reinterpret_cast<lds_u32x2*>(p_hi + off) = u32x2{h0, h1};
        *reinterpret_cast<lds_u32x2*>(p_lo + off) = u32x2{l0, l1};
        if (kg == 0) alpha[hq] = al;
    }

    // O^T += V^T P^T over this wave's value quarter, after rescaling the
    // columns of heads whose reference max moved.  Within each 16-lane block,
    // ds_read_b64_tr_b16 hands lane i element (i & 3) of the 8-byte chunk
    // addressed by lane (i >> 2) + 4e, e = 0..3: lane s addresses key
    // 4g + (s >> 2), dims dt*16 + 4(s & 3) .. +3, so lane i receives keys
    // 4g + e at dim dt*16 + i (and 16 + 4g + e from the second read).
    __device__ __forceinline__ void pv(const lds_u8* lds, const lds_u8* p_hi, const lds_u8* p_lo, const lds_f32* alpha,
                                       int g, int c16, int q) {
        constexpr int ROWB = Geo<D>::ROWB;
        const float a0 = alpha[c16], a1 = alpha[16 + c16];
        if (__builtin_amdgcn_ballot_w64(a0 != 1.0f || a1 != 1.0f)) {
#pragma unroll
            for (int dt = 0; dt < NDQ; ++dt) {
                o[0][dt] *= a0;
                o[1][dt] *= a1;
            }
        }
        bf16x8 pb[2], pbl[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            pb[hb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const lds_u32x4*>(p_hi + (hb * 16 + c16) * PROW + 16 * g));
            pbl[hb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const lds_u32x4*>(p_lo + (hb * 16 + c16) * PROW + 16 * g));
        }
        const lds_u8* vbase = lds + (4 * g + (c16 >> 2)) * ROWB + q * DVQ * 2 + 8 * (c16 & 3);
        constexpr int G4 = 3;
#pragma unroll
        for (int d0 = 0; d0 < NDQ; d0 += G4) {
            bf16x8 vA[G4];
#pragma unroll
            for (int j = 0; j < G4; ++j) {
                if (d0 + j < NDQ) {
                    const lds_u8* p0 = vbase + (d0 + j) * 32;
                    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
                    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 16 * ROWB));
                    vA[j] = __builtin_bit_cast(
                        bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                                      __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
                }
            }
#pragma unroll
            for (int j = 0; j < G4; ++j)
#pragma unroll
                for (int hb = 0; hb < 2; ++hb)
                    if (d0 + j < NDQ) o[hb][d0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA[j], pb[hb], o[hb][d0 + j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < G4; ++j)
#pragma unroll
                for (int hb = 0; hb < 2; ++hb)
                    if (d0 + j < NDQ) o[hb][d0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA[j], pbl[hb], o[hb][d0 + j], 0, 0, 0);
        }
    }
};

constexpr int kXcds = 8;               // XCDs of the GPU; workgroup ids are dealt to them round-robin
constexpr int kWaves = 8;              // two head groups of 32 x four quarters of D
constexpr int kThreads = kWaves * 64;
constexpr int kBtLds = 4096;           // block-table entries cached in LDS
constexpr int kIdxLds = 2560;          // top-k slots cached in LDS (= max keys per split)

template <int KVD, int WD, int D, int DV>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_mfma_kernel(AttnArgs a) {
    using G = Geo<D>;
    using QW = QuarterWave<D, DV>;
    constexpr int NT = kThreads;
    using TL = Tiler<KVD, WD, D, NT>;
    constexpr int NU = TL::NU;
    // tiles held in registers ahead of the LDS stage
    constexpr int kPrefetch = NU <= 12 ? 2 : 1;
    static_assert(kPrefetch == 1 || kPrefetch == 2, "prefetch depth");
    __shared__ __attribute__((aligned(16))) uint8_t stage[2][G::STAGE];
    __shared__ __attribute__((aligned(16))) float kmeta[2][kKeys];
    __shared__ int32_t bt_mem[kBtLds];
    __shared__ int32_t idx_mem[kIdxLds];
    __shared__ __attribute__((aligned(16))) uint8_t xs_mem[kWaves][QW::XSLOT];     // partial-score exchange
    __shared__ __attribute__((aligned(16))) uint8_t p_mem[2][2][QW::PGRP];        // [head group][hi, lo]
    __shared__ __attribute__((aligned(16))) float alpha_mem[2][32];
    __shared__ float fin_mem[2][2][32];                                           // [head group][m, l][head]
    lds_i32* const bt_lds = (lds_i32*)&bt_mem[0];
    lds_i32* const idx_lds = (lds_i32*)&idx_mem[0];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    // workgroup -> (row, split, head block): workgroups are dispatched to the
    // eight XCDs round-robin by id, so id % 8 picks the XCD, and each XCD
    // takes an equal contiguous range of the (row, split) units in row order;
    // a row's queries then reach one or two L2s instead of all eight, and
    // neighbouring rows (which share most of their window) run side by side
    const int units = a.num_rows * a.nsplit;
    const int upx = (units + kXcds - 1) / kXcds;
    const int xcd = (int)blockIdx.x % kXcds, slot = (int)blockIdx.x / kXcds;
    const int hblk = slot / upx;
    const int unit = xcd * upx + slot % upx;
    if (unit >= units) return;
    const int r = unit / a.nsplit, split = unit % a.nsplit;
    const RowKeys rk = row_keys(a, r);
    const int tb = split * a.split_tiles;
    if (tb >= rk.tiles) {
        // empty split (a row with fewer tiles than the longest): a zero state
        if (a.nsplit > 1 && tid < 64) {
            float* ml = a.part_ml + ((int64_t)r * a.nsplit + split) * 2 * a.H + hblk * 64 + tid;
            ml[0] = -INFINITY;
            ml[a.H] = 0.0f;
        }
        return;
    }
    const int te = min(tb + a.split_tiles, rk.tiles);
    const int hg = wave >> 2, q = wave & 3;
    const int head0 = hblk * 64 + hg * 32;                   // first head of this wave's group

    // prologue: top-k slots and block-table range of this split into LDS
    const int sel_end = min(te, rk.sel_tiles) * kKeys;            // selected slots [tb*32, sel_end)
    const int idx0 = tb * kKeys;
    int blk0 = 0, nblk = 0, bt_first = 0;
    if (sel_end > idx0) {
        const int E = 256 / a.m;
        if (a.topk) {
            nblk = (rk.n + E - 1) / E;
            const int nidx = sel_end - idx0;
            const int first = a.topk[(int64_t)r * a.k + min(idx0 + tid, a.k - 1)];
            bt_first = a.block_table[(int64_t)rk.b * a.max_blocks + min(tid, a.max_blocks - 1)];
            if (tid < nidx) idx_lds[tid] = idx0 + tid < rk.nsel ? first : -1;
            for (int i = tid + NT; i < nidx; i += NT)
                idx_lds[i] = idx0 + i < rk.nsel ? a.topk[(int64_t)r * a.k + idx0 + i] : -1;
        } else {
            const int g1 = min(sel_end, rk.nsel);
            if (g1 > idx0) {
                blk0 = idx0 / E;
                nblk = (g1 - 1) / E - blk0 + 1;
                bt_first = a.block_table[(int64_t)rk.b * a.max_blocks + min(blk0 + tid, a.max_blocks - 1)];
            }
        }
    }
    // (the first slot and block of each thread are requested together above,
    // so the common case costs one round trip)
    const int nbt = min(nblk, kBtLds);
    if (tid < nbt) bt_lds[tid] = bt_first;
    for (int i = tid + NT; i < nbt; i += NT) bt_lds[i] = a.block_table[(int64_t)rk.b * a.max_blocks + blk0 + i];
    __syncthreads();

    QW W;
    W.init(a, r, head0, g, c16, q);
    lds_u8* const xs_mine = (lds_u8*)&xs_mem[wave][0];
    const lds_u8* const xs_grp = (const lds_u8*)&xs_mem[hg * 4][0];
    lds_u8* const p_hi = (lds_u8*)&p_mem[hg][0][0];
    lds_u8* const p_lo = (lds_u8*)&p_mem[hg][1][0];
    lds_f32* const alpha = (lds_f32*)&alpha_mem[hg][0];

    TileRegs<NU> R[kPrefetch];
    const int ntl = te - tb;
    TL::issue(a, TL::resolve(a, rk, tb, true, idx_lds, idx0, bt_lds, blk0), R[0]);
    if constexpr (kPrefetch > 1) TL::issue(a, TL::resolve(a, rk, tb + 1, 1 < ntl, idx_lds, idx0, bt_lds, blk0), R[1]);
    lds_u8* const st = (lds_u8*)&stage[0][0];
    lds_f32* const km = (lds_f32*)&kmeta[0][0];
    TL::store(rk, tb, R[0], st, km);
    TL::issue(a, TL::resolve(a, rk, tb + kPrefetch, kPrefetch < ntl, idx_lds, idx0, bt_lds, blk0), R[0]);
    __syncthreads();

    // tile u sits in register set (u - tb) % P until it is stored to stage
    // (u - tb) % 2; the steps of one round are spelled out so that every
    // register set is addressed statically.  Step t: scores of tile t; a
    // barrier (every wave is past the P V of tile t - 1, so its stage is
    // free); tile t + 1 stored there and the loads of tile t + 1 + P issued;
    // the owner softmax; a barrier; P V of tile t.
    auto step = [&](auto J, int t) __attribute__((always_inline)) {
        constexpr int nxt = (decltype(J)::value + 1) % kPrefetch;
        const lds_u8* cur = st + (t & 1) * G::STAGE;
        W.scores(cur, xs_mine, g, c16);
        // the next loads' storage rows come from LDS before the barrier
        const typename TL::Src nsrc =
            TL::resolve(a, rk, tb + t + 1 + kPrefetch, t + 1 + kPrefetch < ntl, idx_lds, idx0, bt_lds, blk0);
        __syncthreads();
        if (t + 1 < ntl)
            TL::store(rk, tb + t + 1, R[nxt], st + ((t + 1) & 1) * G::STAGE, km + ((t + 1) & 1) * kKeys);
        TL::issue(a, nsrc, R[nxt]);
        W.softmax(xs_grp, km + (t & 1) * kKeys, p_hi, p_lo, alpha, lane, q, a.scale_log2);
        __syncthreads();
        W.pv(cur, p_hi, p_lo, alpha, g, c16, q);
    };
    for (int t0 = 0; t0 < ntl; t0 += kPrefetch) {
        step(IntC<0>{}, t0);
        if constexpr (kPrefetch > 1)
            if (t0 + 1 < ntl) step(IntC<1>{}, t0 + 1);
    }

    // finish: each owner's row sum over its eight lanes, published with the
    // reference max for the waves that hold the heads' value columns
    {
        float l_tot = W.l_run + __shfl_xor(W.l_run, 8);
        l_tot += __shfl_xor(l_tot, 16);
        l_tot += __shfl_xor(l_tot, 32);
        if (lane < 8) {
            fin_mem[hg][0][8 * q + lane] = W.m_run;
            fin_mem[hg][1][8 * q + lane] = l_tot;
        }
    }
    __syncthreads();
    constexpr int NDQ = QW::NDQ;
    const int dv0 = q * QW::DVQ + 4 * g;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        const int hl = 16 * hb + c16, hd = head0 + hl;
        const float m_tot = fin_mem[hg][0][hl], l_tot = fin_mem[hg][1][hl];
        if (a.nsplit == 1) {
            const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            const int64_t base = ((int64_t)r * a.H + hd) * DV + dv0;
            if (a.out_dtype == DT_F32) {
                float* out = reinterpret_cast<float*>(a.out) + base;
#pragma unroll
                for (int dt = 0; dt < NDQ; ++dt) *reinterpret_cast<f32x4*>(out + dt * 16) = W.o[hb][dt] * inv;
            } else {
                uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + base;
#pragma unroll
                for (int dt = 0; dt < NDQ; ++dt) {
                    f32x4 t = W.o[hb][dt] * inv;
                    *reinterpret_cast<u32x2*>(out + dt * 16) = u32x2{cvt_pk_bf16(t[0], t[1]), cvt_pk_bf16(t[2], t[3])};
                }
            }
            if (a.lse && g == 0 && q == 0) a.lse[(int64_t)r * a.H + hd] = (m_tot + log2f(l_tot)) * kLn2;
        } else if (a.part_h) {
            // U = O / l, a convex combination of the values, as fp16 scaled
            // by 2^(15 - e) where max |U| over the head's quarter < 2^e
            const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            float amax = 0.0f;
#pragma unroll
            for (int dt = 0; dt < NDQ; ++dt)
#pragma unroll
                for (int v = 0; v < 4; ++v) amax = fmaxf(amax, fabsf(W.o[hb][dt][v]));
            amax *= inv;
            amax = fmaxf(amax, __shfl_xor(amax, 16));
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            int ex = 0;
            (void)frexpf(amax, &ex);
            const float sc = ldexpf(inv, 15 - ex);
            uint16_t* ph = a.part_h + (((int64_t)r * a.nsplit + split) * a.H + hd) * DV + dv0;
#pragma unroll
            for (int dt = 0; dt < NDQ; ++dt) {
                const f32x4 t = W.o[hb][dt] * sc;
                *reinterpret_cast<u32x2*>(ph + dt * 16) = u32x2{pack_f16x2(t[0], t[1]), pack_f16x2(t[2], t[3])};
            }
            if (g == 0) a.part_sc[(((int64_t)r * a.nsplit + split) * 4 + q) * a.H + hd] = ldexpf(1.0f, ex - 15);
            if (g == 0 && q == 0) {
                float* ml = a.part_ml + ((int64_t)r * a.nsplit + split) * 2 * a.H;
                ml[hd] = m_tot;
                ml[a.H + hd] = l_tot;
            }
        } else {
            float* po = a.part_o + (((int64_t)r * a.nsplit + split) * a.H + hd) * DV + dv0;
#pragma unroll
            for (int dt = 0; dt < NDQ; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = W.o[hb][dt];
            if (g == 0 && q == 0) {
                float* ml = a.part_ml + ((int64_t)r * a.nsplit + split) * 2 * a.H;
                ml[hd] = m_tot;
                ml[a.H + hd] = l_tot;
            }
        }
    }
}

// Merge the key splits of one (row, head): m* = max m_s, w_s = 2^(m_s - m*),
// out = sum_s w_s O_s / sum_s w_s l_s, lse = (m* + log2 sum_s w_s l_s) ln 2.
// With fp16 partials (HALF) a split stores U_s = O_s / l_s scaled by a power
// of two per quarter of the value dims, so its weight in the sum becomes
// w_s l_s times that scale.  Each thread owns 4 value dims.  The partial
// outputs of the first MB splits (MB = 16, or 64 for more than 16 splits)
// are requested before anything else, so they are in flight while the block
// forms the weights (thread s owns split s and s + kMergeThreads); loads past
// the last split are not issued.  Empty splits carry m = -inf, weight 0, and
// their workspace bytes are never used.
constexpr int kMergeThreads = 192;     // >= 576 / 4
constexpr int kMaxSplits = 256;        // <= 2 * kMergeThreads

template <bool HALF>
struct MergePart {
    typedef typename std::conditional<HALF, u32x2, f32x4>::type raw;
    __device__ __forceinline__ static raw load(const AttnArgs& a, int64_t off) {
        if constexpr (HALF) return *reinterpret_cast<const u32x2*>(a.part_h + off);
        else return *reinterpret_cast<const f32x4*>(a.part_o + off);
    }
    __device__ __forceinline__ static f32x4 value(const raw& x) {
        if constexpr (HALF) return f32x4{f16_lo(x[0]), f16_hi(x[0]), f16_lo(x[1]), f16_hi(x[1])};
        else return x;
    }
};

template <bool HALF, int MB>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(AttnArgs a) {
    __shared__ float wts[kMaxSplits];
    __shared__ float red[2][kMergeThreads / 64];
    using MP = MergePart<HALF>;
    const int h = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
    const int H = a.H, DV = a.d_v, ns = a.nsplit;
    const float* ml = a.part_ml + (int64_t)r * ns * 2 * H + h;
    const int d = 4 * tid;
    const bool mine = d < DV;
    const int64_t pbase = ((int64_t)r * ns * H + h) * DV + (mine ? d : 0);
    const int64_t sstride = (int64_t)H * DV;
    // fp16 partials: this thread's quarter of the value dims picks the scale
    const float* scp = HALF ? a.part_sc + ((int64_t)r * ns * 4 + (mine ? d / (DV / 4) : 0)) * H + h : nullptr;
    typename MP::raw os[MB];
    float sc[HALF ? MB : 1];
#pragma unroll
    for (int j = 0; j < MB; ++j) {
        if (j < ns) {
            os[j] = MP::load(a, pbase + j * sstride);
            if constexpr (HALF) sc[j] = scp[(int64_t)j * 4 * H];
        }
    }
    const int s1 = tid + kMergeThreads;
    const float m0 = tid < ns ? ml[(int64_t)tid * 2 * H] : -INFINITY;
    const float l0 = tid < ns ? ml[(int64_t)tid * 2 * H + H] : 0.0f;
    const float m1 = s1 < ns ? ml[(int64_t)s1 * 2 * H] : -INFINITY;
    const float l1 = s1 < ns ? ml[(int64_t)s1 * 2 * H + H] : 0.0f;
    float M = wave_max(fmaxf(m0, m1));
    if ((tid & 63) == 0) red[0][tid >> 6] = M;
    __syncthreads();
    M = red[0][0];
#pragma unroll
    for (int i = 1; i < kMergeThreads / 64; ++i) M = fmaxf(M, red[0][i]);
    const float w0 = m0 == -INFINITY ? 0.0f : exp2f(m0 - M);
    const float w1 = m1 == -INFINITY ? 0.0f : exp2f(m1 - M);
    // fp16 partials are normalised, so their weight carries l_s
    if (tid < ns) wts[tid] = HALF ? w0 * l0 : w0;
    if (s1 < ns) wts[s1] = HALF ? w1 * l1 : w1;
    float L = wave_sum(w0 * l0 + w1 * l1);
    if ((tid & 63) == 0) red[1][tid >> 6] = L;
    __syncthreads();
    L = 0.0f;
#pragma unroll
    for (int i = 0; i < kMergeThreads / 64; ++i) L += red[1][i];
    if (a.lse && tid == 0) a.lse[(int64_t)r * H + h] = (M + log2f(L)) * kLn2;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    auto add = [&](int s, int j) __attribute__((always_inline)) {
        const float w = s < ns ? wts[s] : 0.0f;
        const float ws = HALF ? w * sc[HALF ? j : 0] : w;
        acc = w > 0.0f ? acc + ws * MP::value(os[j]) : acc;
    };
#pragma unroll
    for (int j = 0; j < MB; ++j)
        if (j < ns) add(j, j);
    for (int s0 = MB; s0 < ns; s0 += MB) {
#pragma unroll
        for (int j = 0; j < MB; ++j) {
            if (s0 + j < ns) {
                os[j] = MP::load(a, pbase + (s0 + j) * sstride);
                if constexpr (HALF) sc[j] = scp[(int64_t)(s0 + j) * 4 * H];
            }
        }
#pragma unroll
        for (int j = 0; j < MB; ++j)
            if (s0 + j < ns) add(s0 + j, j);
    }
    if (!mine) return;
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    acc *= inv;
    const int64_t oi = ((int64_t)r * H + h) * DV + d;
    if (a.out_dtype == DT_F32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + oi) = acc;
    } else {
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + oi) =
            u32x2{cvt_pk_bf16(acc[0], acc[1]), cvt_pk_bf16(acc[2], acc[3])};
    }
}

// fp32 path (tiny workloads): one workgroup per (row, head); scores in LDS.
constexpr int kF32MaxKeys = 8192;
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
    __shared__ float sc[kF32MaxKeys];
    __shared__ float red[4];
    const int h = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
    const int b = a.row_seq[r], p = a.row_pos[r];
    const int n = visible_entries(p, a.m);
    const int nsel = a.topk ? a.k : n;
    const int t0 = max(0, p - a.window + 1);
    const int L = nsel + (p - t0 + 1);
    const int E = 256 / a.m;
    const int D = a.D;
    const float* q = reinterpret_cast<const float*>(a.q) + ((int64_t)r * a.H + h) * D;
    const float* kvd = reinterpret_cast<const float*>(a.kv_data);
    const float* wd = reinterpret_cast<const float*>(a.win_data);
    const float scale = a.scale_log2 * kLn2;
    auto key_ptr = [&](int j) -> const float* {
        if (j < nsel) {
            const int g = a.topk ? a.topk[(int64_t)r * a.k + j] : j;
            if (g < 0 || g >= n) return nullptr;
            return kvd + ((int64_t)a.block_table[(int64_t)b * a.max_blocks + g / E] * E + g % E) * D;
        }
        return wd + ((int64_t)b * a.win_cap + (t0 + j - nsel) % a.win_cap) * D;
    };
    float mx = -INFINITY;
    for (int j = tid; j < L; j += 256) {
        const float* kp = key_ptr(j);
        float s = -INFINITY;
        if (kp) {
            float dot = 0.0f;
            for (int d = 0; d < D; ++d) dot = fmaf(q[d], kp[d], dot);
            s = scale * dot;
        }
        sc[j] = s;
        mx = fmaxf(mx, s);
    }
    mx = wave_max(mx);
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float sum = 0.0f;
    for (int j = tid; j < L; j += 256) {
        float e = sc[j] == -INFINITY ? 0.0f : expf(sc[j] - mx);
        sc[j] = e;
        sum += e;
    }
    sum = wave_sum(sum);
    if ((tid & 63) == 0) red[tid >> 6] = sum;
    __syncthreads();
    sum = red[0] + red[1] + red[2] + red[3];
    const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
    for (int d = tid; d < a.d_v; d += 256) {
        float acc = 0.0f;
        for (int j = 0; j < L; ++j) {
            if (sc[j] == 0.0f) continue;
            acc = fmaf(sc[j], key_ptr(j)[d], acc);
        }
        const int64_t oi = ((int64_t)r * a.H + h) * a.d_v + d;
        if (a.out_dtype == DT_F32) reinterpret_cast<float*>(a.out)[oi] = acc * inv;
        else reinterpret_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16(acc * inv);
    }
    if (a.lse && tid == 0) a.lse[(int64_t)r * a.H + h] = mx + logf(sum);
}

template <int KVD, int WD, int D, int DV>
hipError_t launch_mfma(const AttnArgs& a, hipStream_t stream) {
    const int64_t upx = ((int64_t)a.num_rows * a.nsplit + kXcds - 1) / kXcds;
    const dim3 grid((unsigned)(kXcds * upx * (a.H / 64)));
    hipLaunchKernelGGL((attn_mfma_kernel<KVD, WD, D, DV>), grid, dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    const dim3 mgrid(a.H, a.num_rows);
    if (a.part_h) {
        if (a.nsplit <= 16) hipLaunchKernelGGL((attn_merge_kernel<true, 16>), mgrid, dim3(kMergeThreads), 0, stream, a);
        else hipLaunchKernelGGL((attn_merge_kernel<true, 64>), mgrid, dim3(kMergeThreads), 0, stream, a);
    } else {
        if (a.nsplit <= 16) hipLaunchKernelGGL((attn_merge_kernel<false, 16>), mgrid, dim3(kMergeThreads), 0, stream, a);
        else hipLaunchKernelGGL((attn_merge_kernel<false, 64>), mgrid, dim3(kMergeThreads), 0, stream, a);
    }
    return hipGetLastError();
}

// Workgroups cover 64 heads (two groups of 32); more heads add head groups
// to the grid.
template <int KVD, int WD, int D, int DV>
hipError_t launch_heads(const AttnArgs& a, hipStream_t stream) {
    if (a.H % 64 != 0) return hipErrorInvalidValue;
    return launch_mfma<KVD, WD, D, DV>(a, stream);
}

template <int KVD, int WD>
hipError_t launch_dims(const AttnArgs& a, hipStream_t stream) {
    if (a.D == 576 && a.d_v == 576) return launch_heads<KVD, WD, 576, 576>(a, stream);
    if (a.D == 576 && a.d_v == 512) return launch_heads<KVD, WD, 576, 512>(a, stream);
    if (a.D == 128 && a.d_v == 128) return launch_heads<KVD, WD, 128, 128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace

int attn_f32_max_keys() { return kF32MaxKeys; }
int attn_max_split_tiles() { return kIdxLds / kKeys; }
int attn_max_splits() { return kMaxSplits; }
int attn_tile_keys() { return kKeys; }
int attn_max_table_blocks() { return kBtLds; }

bool attn_supported(int q_dtype, int kv_dtype, int win_dtype, int H, int D, int d_v) {
    if (q_dtype == DT_F32)
        return kv_dtype == DT_F32 && (win_dtype == DT_F32 || win_dtype == DT_NONE) && D >= 1 && d_v <= D;
    if (q_dtype != DT_BF16) return false;
    if (kv_dtype != DT_BF16 && kv_dtype != DT_MXFP4) return false;
    if (win_dtype != DT_BF16 && win_dtype != DT_FP8) return false;
    if (H < 64 || H % 64 != 0) return false;
    return (D == 576 && (d_v == 576 || d_v == 512)) || (D == 128 && d_v == 128);
}

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream) {
    if (a.num_rows <= 0) return hipSuccess;
    if (a.kv_dtype == DT_F32) {
        hipLaunchKernelGGL(attn_f32_kernel, dim3(a.H, a.num_rows), dim3(256), 0, stream, a);
        return hipGetLastError();
    }
    if (a.kv_dtype == DT_BF16 && a.win_dtype == DT_FP8) return launch_dims<DT_BF16, DT_FP8>(a, stream);
    if (a.kv_dtype == DT_BF16 && a.win_dtype == DT_BF16) return launch_dims<DT_BF16, DT_BF16>(a, stream);
    if (a.kv_dtype == DT_MXFP4 && a.win_dtype == DT_FP8) return launch_dims<DT_MXFP4, DT_FP8>(a, stream);
    if (a.kv_dtype == DT_MXFP4 && a.win_dtype == DT_BF16) return launch_dims<DT_MXFP4, DT_BF16>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace lcca
