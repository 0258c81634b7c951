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
// bf16/MFMA path.  A workgroup = (row, range of key tiles, group of 64
// heads), eight waves, two per SIMD:
//   prologue: the storage row of every selected slot of the split is resolved
//     through the top-k list and the block table once, into LDS;
//   loads:    the four score waves load each tile's raw bytes (bf16, FP8 or
//     MXFP4 + E8M0 scales) into registers two tiles ahead, convert them
//     exactly to bf16 and write them to one of three padded LDS stages; one
//     barrier per tile;
//   scores:   each score wave holds 16 heads' queries over all of D and forms
//     S^T = K Q^T for the tile with MFMA 16x16x32 (A = keys from LDS), the
//     online softmax in the exp2 domain in registers, and P as a bf16 hi + lo
//     pair (16 significant bits) into LDS; FP8 window scales multiply the
//     scores and are folded into P;
//   values:   each value wave holds the O^T accumulators of all 64 heads over
//     a quarter of the value dims and runs O^T += V^T P^T with V^T read from
//     the same LDS tile by ds_read_b64_tr_b16 (K = V), one tile behind the
//     score waves.
// FP8 queries on MXFP4 pools: each head's query is quantised to E4M3 with a
// power-of-two scale; the loaders also keep each pool tile's E2M1 codes and
// E8M0 scales as stored (two raw stages), and the score waves form S^T from
// them with the scaled 16x16x128 FP4 x FP8 MFMA; window tiles use bf16 MFMAs
// on the dequantised query.  The value side is unchanged.
// Keys are split across workgroups when the rows alone cannot fill the GPU;
// the partial (max, sum, O) states go to the workspace and a merge kernel
// (one workgroup per row and 16 value dims) combines them.  For fp32 outputs
// O stays fp32; for bf16 outputs O / sum is stored as fp16 (11 significant
// bits, eight times finer than the output's rounding) with a power-of-two
// range scale per split, head and 4 value dims.
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace lcca {

namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kKeys = 32;              // keys per tile
constexpr float kLazy = 16.0f;         // reference-max slack of the online softmax (log2 units)

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

// FP8 queries on MXFP4 pool tiles: the tile's E2M1 codes and E8M0 scales as
// the pool stores them, in a stage of their own (two stages: written one
// step ahead, read only by the score waves in the next step).
template <int D>
struct Raw {
    static constexpr int ROWB = D / 2 + 16;          // codes of a key, padded: 16 lanes' 16-B reads at
                                                     // rows 304 B apart start 12 banks apart (no conflict)
    static constexpr int SCB = D / 32;               // scale bytes of a key
    static constexpr int SC0 = kKeys * ROWB;         // offset of the scale bytes
    static constexpr int STAGE = SC0 + ((kKeys * SCB + 15) & ~15);
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
    k.b = checked(a.row_seq[r], 0, a.batch - 1, a.dbg, kDbgRow);
    k.p = checked(a.row_pos[r], 0, a.max_pos, a.dbg, kDbgRow);
    k.n = visible_entries(k.p, a.m);
    k.nsel = a.topk ? a.k : k.n;
    k.sel_tiles = (k.nsel + kKeys - 1) / kKeys;
    k.t0 = max(0, k.p - a.window + 1);
    k.nwin = k.p - k.t0 + 1;
    k.tiles = k.sel_tiles + (k.nwin + kKeys - 1) / kKeys;
    return k;
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
    // also read row 0 and are zeroed when stored.  rows_lds holds the storage
    // row of every selected slot of the split from idx0 on (-1: masked).
    struct Src {
        int64_t row;
        bool ok, win;
    };
    // The LDS read of the storage row is separate (row_of, issued early;
    // for window tiles its value is not used) from forming the source.
    __device__ __forceinline__ static int row_of(const RowKeys& rk, int tile, bool live, const lds_i32* rows_lds,
                                                 int idx0) {
        const int key = (int)threadIdx.x / kThreadsPerKey;
        return rows_lds[(live && tile < rk.sel_tiles ? tile * kKeys - idx0 : 0) + key];
    }
    __device__ __forceinline__ static Src resolve(const AttnArgs& a, const RowKeys& rk, int tile, bool live,
                                                  int prow) {
        const int key = (int)threadIdx.x / kThreadsPerKey;
        Src s;
        s.win = live && tile >= rk.sel_tiles;                       // uniform over the workgroup
        if (s.win) {
            const int w = (tile - rk.sel_tiles) * kKeys + key;
            s.ok = w < rk.nwin;
            s.row = (int64_t)rk.b * a.win_cap + (rk.t0 + (s.ok ? w : 0)) % a.win_cap;
        } else {
            s.ok = live && prow >= 0;
            s.row = s.ok ? prow : 0;
        }
        return s;
    }
    __device__ __forceinline__ static Src resolve(const AttnArgs& a, const RowKeys& rk, int tile, bool live,
                                                  const lds_i32* rows_lds, int idx0) {
        return resolve(a, rk, tile, live, row_of(rk, tile, live, rows_lds, idx0));
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

    // FP8-query path: the E2M1 codes and E8M0 scales of a pool tile, as
    // stored (a masked key: zero codes, scale 1).
    __device__ __forceinline__ static void store_raw(const TileRegs<NU>& R, lds_u8* raw) {
        static_assert(KVD == DT_MXFP4, "raw stages hold MXFP4 tiles");
        const int tid = threadIdx.x;
        const int key = tid / kThreadsPerKey, sub = tid % kThreadsPerKey;
        const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < NU_P; ++i) {
            const int part = sub + kThreadsPerKey * i;
            if ((i + 1) * kThreadsPerKey <= UPK_P || part < UPK_P) {
                *reinterpret_cast<lds_u32x4*>(raw + key * Raw<D>::ROWB + part * 16) = R.valid ? R.v[i] : zero;
                raw[Raw<D>::SC0 + key * Raw<D>::SCB + part] = (uint8_t)(R.valid ? R.sc[i] : 127u);
            }
        }
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

// Two kinds of waves share a workgroup (eight waves, two per SIMD):
//   score waves 0..3 each hold the queries of 16 heads over the whole of D in
//     VGPRs (B operands) and run, per 32-key tile, S^T = K Q^T with MFMA
//     16x16x32 (keys on M in two 16-key blocks, heads on N; A = keys from LDS),
//     the online softmax in registers (a lane holds 8 keys of one head: the C
//     layout, keys 4g..4g+3 and 16+4g..16+4g+3, g = lane >> 4), and write P as
//     a bf16 hi + lo pair (16 significant bits) in B-operand order, with each
//     head's rescale factor, to LDS; they also load the key tiles;
//   value waves 4..7 each hold the O^T accumulators of all 64 heads over a
//     quarter of the value dims and run O^T += V^T P^T with MFMA 16x16x32,
//     V^T read from the same LDS tile (K = V) by ds_read_b64_tr_b16 in the key
//     order of the C layout, each V^T fragment feeding the four head blocks.
// Each SIMD hosts one wave of each kind, so the score wave's softmax, loads
// and tile stores overlap the value wave's MFMAs.  One barrier per tile: in
// step k the score waves work on tile k while the value waves finish tile
// k - 1.
template <int D, bool Q8>
struct ScoreWave {
    static constexpr int KS = D / 32;                        // 32-dim k-steps over D
    static constexpr int KS8 = (D + 127) / 128;              // 128-dim k-steps of the FP4 x FP8 MFMA
    bf16x8 qb[Q8 ? 1 : KS];                                  // bf16 queries (B operands)
    i32x8 q8[Q8 ? KS8 : 1];                                  // FP8 query codes (B operands)
    int qx;                                                  // their power-of-two scale X
    float m_run, l_run;                                      // head (lane & 15): reference max, this lane's keys' sum

    __device__ __forceinline__ void init(const AttnArgs& a, int r, int head0, int lane) {
        if constexpr (!Q8) {
            const int c16 = lane & 15, g = lane >> 4;
            const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)r * a.H + head0 + c16) * D + 8 * g;
#pragma unroll
            for (int s = 0; s < KS; ++s)
                qb[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 32 * s));
        } else {
            // The head's query quantised to E4M3 with one power-of-two scale:
            // X = floor(log2 max |q|) - 7 (the maximum / 2^X lands in
            // [128, 256), no saturation; X = -127 for a zero query), codes =
            // RNE(q / 2^X).  B operand of k-step s (scaled 16x16x128 MFMA,
            // FP8): byte e of lane group g is dim 128 s + 16 g + e for e < 16
            // and 128 s + 64 + 16 g + (e - 16) for e >= 16 (dims past D: 0);
            // the four lanes of a head hold all of its dims.
            const int c16 = lane & 15, g = lane >> 4;
            const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)r * a.H + head0 + c16) * D;
            u32x4 v[KS8][2][2];
#pragma unroll
            for (int s = 0; s < KS8; ++s)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        v[s][h][t] = 128 * s + 64 * h < D
                                         ? *reinterpret_cast<const u32x4*>(qrow + 128 * s + 64 * h + 16 * g + 8 * t)
                                         : u32x4{0u, 0u, 0u, 0u};
            float amax = 0.0f;
#pragma unroll
            for (int s = 0; s < KS8; ++s)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            amax = fmaxf(amax, fmaxf(fabsf(bf16_to_f32(v[s][h][t][j] & 0xffffu)),
                                                     fabsf(bf16_to_f32(v[s][h][t][j] >> 16))));
            amax = fmaxf(amax, __shfl_xor(amax, 16));
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            int X = -127;
            if (amax > 0.0f) {
                int ex = 0;
                (void)frexpf(amax, &ex);
                X = min(max(ex - 8, -127), 127);
            }
            qx = X;
            // q / 2^X is exact (a power of two; |q / 2^X| < 256); the
            // hardware conversion rounds to nearest even, the same codes as
            // the library's software encoder for every bf16 value below 448
            const float inv = ldexpf(1.0f, -X);
#pragma unroll
            for (int s = 0; s < KS8; ++s) {
                uint32_t w[8];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            const uint32_t u0 = v[s][h][t][2 * j], u1 = v[s][h][t][2 * j + 1];
                            int c = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_to_f32(u0 & 0xffffu) * inv,
                                                                    bf16_to_f32(u0 >> 16) * inv, 0, false);
                            c = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_to_f32(u1 & 0xffffu) * inv,
                                                                bf16_to_f32(u1 >> 16) * inv, c, true);
                            w[4 * h + 2 * t + j] = (uint32_t)c;
                        }
                q8[s] = i32x8{(int)w[0], (int)w[1], (int)w[2], (int)w[3], (int)w[4], (int)w[5], (int)w[6], (int)w[7]};
            }
        }
        m_run = -INFINITY;
        l_run = 0.0f;
    }

    // S^T of a pool tile from its raw stage (FP8 queries): the scaled
    // 16x16x128 MFMA with A = the keys' E2M1 codes, lane (key k16, g) holding
    // MX block 4s + g (32 dims, its own E8M0 scale) and B = the FP8 query
    // codes with the head's scale.  Same C layout as scores().
    __device__ __forceinline__ void scores8(const lds_u8* raw, int lane, f32x4 (&sacc)[2]) const {
        using RG = Raw<D>;
        const int k16 = lane & 15, g = lane >> 4;
        sacc[0] = sacc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const lds_u8* kr = raw + (16 * b + k16) * RG::ROWB + 16 * g;
            const lds_u8* ks = raw + RG::SC0 + (16 * b + k16) * RG::SCB + g;
#pragma unroll
            for (int s = 0; s < KS8; ++s) {
                constexpr int kBlocks = D / 32;
                const bool in = 4 * s + g < kBlocks;
                u32x4 v = u32x4{0u, 0u, 0u, 0u};
                int sa = 127;
                if (in) {
                    v = *reinterpret_cast<const lds_u32x4*>(kr + 64 * s);
                    sa = ks[4 * s];
                }
                const i32x8 av = i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
                sacc[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, q8[s], sacc[b], 4, 0, 0, sa, 0,
                                                                          qx + 127);
            }
        }
    }

    // S^T of a window tile (bf16 LDS stage) with FP8 queries: bf16 MFMAs on
    // the dequantised query code * 2^X (exact in bf16), formed from the codes
    // per k-step, dims assigned to lanes as in the codes: k-step (s, t), lane
    // group g takes dims 128 s + 64 (t >> 1) + 16 g + 8 (t & 1) .. +7 for
    // both operands.
    __device__ __forceinline__ void scores_q8win(const lds_u8* st, int lane, f32x4 (&sacc)[2]) const {
        constexpr int ROWB = Geo<D>::ROWB;
        const int g = lane >> 4;
        const lds_u8* kb = st + (lane & 15) * ROWB + 32 * g;
        const float sc = ldexpf(1.0f, qx);
        sacc[0] = sacc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS8; ++s) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (128 * s + 64 * (t >> 1) >= D) continue;
                uint32_t w0 = (uint32_t)q8[s][4 * (t >> 1) + 2 * (t & 1)];
                uint32_t w1 = (uint32_t)q8[s][4 * (t >> 1) + 2 * (t & 1) + 1];
                // formed per tile: hoisted out of the tile loop, the 72
                // registers of the bf16 query would stay live beside the codes
                asm volatile("" : "+v"(w0), "+v"(w1));
                const bf16x8 qv = __builtin_bit_cast(
                    bf16x8, u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false)),
                                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true)),
                                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false)),
                                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true))});
                const int off = 2 * (128 * s + 64 * (t >> 1) + 8 * (t & 1));
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const bf16x8 k = __builtin_bit_cast(bf16x8, *reinterpret_cast<const lds_u32x4*>(kb + 16 * b * ROWB + off));
                    sacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k, qv, sacc[b], 0, 0, 0);
                }
            }
        }
    }

    // S^T of the tile: lane (head = lane & 15, g = lane >> 4) gets keys
    // 16 b + 4g + j in sacc[b][j].
    // The K fragments are read in batches of KB k-steps, the next batch's
    // reads issued before the current batch's MFMAs, so LDS latency overlaps
    // the MFMAs instead of gating each of them.
    template <int KB>
    __device__ __forceinline__ void scores(const lds_u8* st, int lane, f32x4 (&sacc)[2]) const {
        constexpr int ROWB = Geo<D>::ROWB;
        constexpr int NB = (KS + KB - 1) / KB;
        const lds_u8* kb = st + (lane & 15) * ROWB + 16 * (lane >> 4);
        sacc[0] = sacc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x8 kf[2][KB][2];
        auto fetch = [&](int buf, int s0) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < KB; ++j)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    if (s0 + j < KS)
                        kf[buf][j][b] = __builtin_bit_cast(
                            bf16x8, *reinterpret_cast<const lds_u32x4*>(kb + 16 * b * ROWB + 64 * (s0 + j)));
        };
        fetch(0, 0);
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            if (n + 1 < NB) fetch((n + 1) & 1, (n + 1) * KB);
            // the scheduler would otherwise sink each read next to its MFMA
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < KB; ++j)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    if (n * KB + j < KS)
                        sacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[n & 1][j][b], qb[n * KB + j], sacc[b], 0, 0, 0);
        }
    }

    // Online softmax of the tile (this lane: 8 keys of one head).  kmeta[key]:
    // the key's value scale (FP8 window scale, 1, or -1 for a masked key),
    // which also multiplies its score.  Returns the rescale factor of the
    // head's accumulators and P hi / lo in B-operand order.
    __device__ __forceinline__ float softmax(f32x4 (&s)[2], const f32x4 (&km)[2], float scale_log2, u32x4& h,
                                             u32x4& l) {
        float mx = -INFINITY;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s[b][j] = km[b][j] >= 0.0f ? s[b][j] * (scale_log2 * km[b][j]) : -INFINITY;
                mx = fmaxf(mx, s[b][j]);
            }
        }
        mx = max_across_rows(mx);
        // Lazy rescaling: the reference max moves only when the tile's max
        // exceeds it by more than kLazy (log2 units); weights relative to it
        // stay below 2^kLazy, far inside fp32 and bf16 range.
        float al = 1.0f;
        if (mx > m_run + kLazy) {
            al = exp2f(m_run - mx);          // 0 while m_run = -inf
            l_run *= al;
            m_run = mx;
        }
        const float mref = m_run == -INFINITY ? 0.0f : m_run;
        float psum = 0.0f;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                // x - mref <= kLazy: v_exp_f32 directly (results below 2^-126
                // may flush to zero, far below the sum's precision)
                const float p0 = __builtin_amdgcn_exp2f(s[b][2 * t] - mref);
                const float p1 = __builtin_amdgcn_exp2f(s[b][2 * t + 1] - mref);
                psum += p0 + p1;
                // masked keys: p = 0; FP8 window keys carry their scale
                const float a0 = p0 * km[b][2 * t], a1 = p1 * km[b][2 * t + 1];
                const uint32_t hh = cvt_pk_bf16(a0, a1);
                h[2 * b + t] = hh;
                l[2 * b + t] = cvt_pk_bf16(a0 - __uint_as_float(hh << 16), a1 - __uint_as_float(hh & 0xffff0000u));
            }
        }
        l_run += psum;
        return al;
    }
};

template <int D, int DV>
struct ValueWave {
    static constexpr int DVQ = DV / 4;                       // value dims per wave
    static constexpr int NDT = DVQ / 16;                     // 16-dim tiles of O^T per head block
    static_assert(DV % 64 == 0, "shape");
    f32x4 o[4][NDT];                                         // [head block][dim tile]
    int vbase;

    __device__ __forceinline__ void init(int q) {
        vbase = q * DVQ;
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) o[hb][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // O^T += V^T P^T over this wave's value quarter for the four head blocks.
    // Within each 16-lane block, ds_read_b64_tr_b16 hands lane i element
    // (i & 3) of the 8-byte chunk addressed by lane (i >> 2) + 4e, e = 0..3;
    // lane s of block g addresses key 4g + (s >> 2) (+ 16 for the second
    // read), dims 16 dt + 4 (s & 3) .. +3 of the quarter, so lane i receives
    // dim 16 dt + i for keys 4g + e and 16 + 4g + e: the A operand of a
    // 16x16x32 MFMA in the key order of the score waves' C layout.
    template <bool LO>
    __device__ __forceinline__ void pv(const lds_u8* st, const bf16x8 (&phi)[4], const bf16x8 (&plo)[4], int lane) {
        constexpr int ROWB = Geo<D>::ROWB;
        const int g = lane >> 4, i16 = lane & 15;
        const lds_u8* vb = st + (4 * g + (i16 >> 2)) * ROWB + (vbase + 4 * (i16 & 3)) * 2;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const lds_u8* p0 = vb + 32 * dt;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 16 * ROWB));
            const bf16x8 va = __builtin_bit_cast(
                bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                              __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) {
                o[hb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi[hb], o[hb][dt], 0, 0, 0);
                if constexpr (LO) o[hb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo[hb], o[hb][dt], 0, 0, 0);
            }
        }
    }
};

constexpr int kXcds = 8;               // XCDs of the GPU; workgroup ids are dealt to them round-robin
constexpr int kWaves = 8;              // four score waves, four value waves
constexpr int kThreads = kWaves * 64;
constexpr int kLoadThreads = 256;      // the score waves load the key tiles
constexpr int kStages = 3;             // LDS stages of the key tiles
constexpr int kRowsLds = 2560;         // storage rows of a split's selected slots cached in LDS (= max keys per split)

// PLO: P enters P.V as a bf16 hi + lo pair (the default) or as bf16 alone.
template <int KVD, int WD, int D, int DV, bool Q8, bool PLO>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_mfma_kernel(AttnArgs a) {
    using G = Geo<D>;
    using SW = ScoreWave<D, Q8>;
    using VW = ValueWave<D, DV>;
    using TL = Tiler<KVD, WD, D, kLoadThreads>;
    constexpr int NU = TL::NU;
    constexpr int NT = kThreads;
    // k-steps of K fragments read ahead of the score MFMAs (two where the
    // bf16 window tiles' load registers leave less room)
    constexpr int KBatch = (KVD == DT_MXFP4 && WD == DT_BF16) ? 2 : 3;
    __shared__ __attribute__((aligned(16))) uint8_t stage[kStages][G::STAGE];
    __shared__ __attribute__((aligned(16))) float kmeta[kStages][kKeys];
    __shared__ __attribute__((aligned(16))) uint8_t p_mem[2][2][4][64 * 16];   // [step parity][hi, lo][head block][lane]
    __shared__ __attribute__((aligned(16))) float al_mem[2][64];                 // [step parity][head]
    __shared__ float fin_mem[2][64];                                              // [m, l][head]
    __shared__ int32_t rows_mem[kRowsLds];
    __shared__ __attribute__((aligned(128))) uint8_t raw_mem[Q8 ? 2 * Raw<D>::STAGE : 16];
    lds_i32* const rows_lds = (lds_i32*)&rows_mem[0];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
            float* ml = a.part_ml + (((int64_t)r * a.nsplit + split) * a.H + hblk * 64 + tid) * 2;
            *reinterpret_cast<float2*>(ml) = float2{-INFINITY, 0.0f};
        }
        return;
    }
    const int te = min(tb + a.split_tiles, rk.tiles);
    const int ntl = te - tb;
    const int head0 = hblk * 64;

    // prologue: the storage row of every selected slot of this split (-1:
    // masked), resolved through the top-k list and the block table once,
    // into LDS; each thread requests all of its slots' loads before waiting
    const int idx0 = tb * kKeys;
    const int nslots = max(0, min(te, rk.sel_tiles) * kKeys - idx0);
    {
        constexpr int kPer = kRowsLds / NT;
        const int sh = __builtin_ctz(256 / a.m);             // E = 256/m entries per block, a power of two
        int gs[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int j = idx0 + tid + NT * i;
            gs[i] = -1;
            if (tid + NT * i < nslots && j < rk.nsel) gs[i] = a.topk ? a.topk[(int64_t)r * a.k + j] : j;
        }
        int pbs[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const bool ok = gs[i] >= 0 && gs[i] < rk.n;
            pbs[i] = ok ? checked(a.block_table[(int64_t)rk.b * a.max_blocks + (gs[i] >> sh)], 0, a.n_blocks - 1,
                                  a.dbg, kDbgBlock)
                        : -1;
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            if (tid + NT * i < nslots) {
                const bool ok = gs[i] >= 0 && gs[i] < rk.n;
                rows_lds[tid + NT * i] = ok ? (pbs[i] << sh) | (gs[i] & ((1 << sh) - 1)) : -1;
            }
        }
    }
    __syncthreads();
    lds_u8* const st = (lds_u8*)&stage[0][0];
    lds_f32* const km = (lds_f32*)&kmeta[0][0];
    lds_u8* const pm = (lds_u8*)&p_mem[0][0][0][0];
    lds_f32* const alm = (lds_f32*)&al_mem[0][0];
    lds_u8* const rw = (lds_u8*)&raw_mem[0];
    constexpr int PPAR = 2 * 4 * 64 * 16;                    // bytes between the two P parities
    const int c16 = lane & 15, g = lane >> 4;

    if (wave < 4) {
        // ---- score waves: head block `wave`, and the key tile loads ----
        const int hb = wave;
        SW W;
        W.init(a, r, head0 + 16 * hb, lane);
        // tile 0 into stage 0; tiles 1 and 2 in flight in the two register sets
        TileRegs<NU> R[2];
        TL::issue(a, TL::resolve(a, rk, tb, true, rows_lds, idx0), R[0]);
        TL::issue(a, TL::resolve(a, rk, tb + 1, 1 < ntl, rows_lds, idx0), R[1]);
        TL::store(rk, tb, R[0], st, km);
        if constexpr (Q8)
            if (tb < rk.sel_tiles) TL::store_raw(R[0], rw);
        TL::issue(a, TL::resolve(a, rk, tb + 2, 2 < ntl, rows_lds, idx0), R[0]);
        __syncthreads();
        // step k: scores, softmax and P of tile k (stage k % 3); register set
        // (k + 1) & 1 (tile k + 1) into stage (k + 1) % 3, which the value
        // waves left in step k - 1, and the loads of tile k + 3 into it; then
        // the barrier.  Register sets are addressed statically (unrolled by two).
        auto step = [&](auto J, int k) __attribute__((always_inline)) {
            constexpr int rs = (decltype(J)::value + 1) & 1;
            const int sc = k % kStages, sn = (k + 1) % kStages;
            // LDS reads whose results are needed only after the scores: the
            // storage row of tile k + 3 and the keys' metadata
            const int nrow = TL::row_of(rk, tb + k + 3, k + 3 < ntl, rows_lds, idx0);
            f32x4 kmv[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) kmv[b] = *reinterpret_cast<const lds_f32x4*>(km + sc * kKeys + 16 * b + 4 * g);
            f32x4 sv[2];
            if constexpr (Q8) {
                if (tb + k < rk.sel_tiles) W.scores8(rw + (k & 1) * Raw<D>::STAGE, lane, sv);
                else W.scores_q8win(st + sc * G::STAGE, lane, sv);
            } else {
                W.template scores<KBatch>(st + sc * G::STAGE, lane, sv);
            }
            const typename TL::Src nsrc = TL::resolve(a, rk, tb + k + 3, k + 3 < ntl, nrow);
            u32x4 h, l;
            const float al = W.softmax(sv, kmv, a.scale_log2, h, l);
            lds_u8* pw = pm + (k & 1) * PPAR + hb * 1024 + lane * 16;
            *reinterpret_cast<lds_u32x4*>(pw) = h;
            if constexpr (PLO) *reinterpret_cast<lds_u32x4*>(pw + 4096) = l;
            if (g == 0) alm[(k & 1) * 64 + 16 * hb + c16] = al;
            if (k + 1 < ntl) {
                TL::store(rk, tb + k + 1, R[rs], st + sn * G::STAGE, km + sn * kKeys);
                if constexpr (Q8)
                    if (tb + k + 1 < rk.sel_tiles) TL::store_raw(R[rs], rw + ((k + 1) & 1) * Raw<D>::STAGE);
            }
            TL::issue(a, nsrc, R[rs]);
            __syncthreads();
        };
        for (int k0 = 0; k0 < ntl; k0 += 2) {
            step(IntC<0>{}, k0);
            if (k0 + 1 < ntl) step(IntC<1>{}, k0 + 1);
        }
        __syncthreads();                                     // the value waves finish the last tile
        // the row sum of each head over all lanes' keys, with its reference max
        float l_tot = W.l_run + __shfl_xor(W.l_run, 16);
        l_tot += __shfl_xor(l_tot, 32);
        const int hd = head0 + 16 * hb + c16;
        if (g == 0) {
            fin_mem[0][16 * hb + c16] = W.m_run;
            fin_mem[1][16 * hb + c16] = l_tot;
            if (a.nsplit == 1) {
                if (a.lse) a.lse[(int64_t)r * a.H + hd] = (W.m_run + log2f(l_tot)) * kLn2;
            } else {
                float* ml = a.part_ml + (((int64_t)r * a.nsplit + split) * a.H + hd) * 2;
                *reinterpret_cast<float2*>(ml) = float2{W.m_run, l_tot};
            }
        }
        __syncthreads();
        return;
    }

    // ---- value waves: quarter `wave - 4` of the value dims, all 64 heads ----
    VW V;
    V.init(wave - 4);
    __syncthreads();                                         // tile 0 in stage 0
    // step k: the score waves' tile k; here P V of tile k - 1 (stage
    // (k - 1) % 3, P of parity (k - 1) & 1); then the barrier
    for (int k = 0; k < ntl; ++k) {
        if (k > 0) {
            const int kp = k - 1;
            bf16x8 phi[4], plo[4];
            const lds_u8* pr = pm + (kp & 1) * PPAR + lane * 16;
            float al[4];
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) {
                phi[hb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const lds_u32x4*>(pr + hb * 1024));
                if constexpr (PLO)
                    plo[hb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const lds_u32x4*>(pr + 4096 + hb * 1024));
                al[hb] = alm[(kp & 1) * 64 + 16 * hb + c16];
            }
            if (__builtin_amdgcn_ballot_w64(al[0] != 1.0f || al[1] != 1.0f || al[2] != 1.0f || al[3] != 1.0f)) {
#pragma unroll
                for (int hb = 0; hb < 4; ++hb)
#pragma unroll
                    for (int dt = 0; dt < VW::NDT; ++dt) V.o[hb][dt] *= al[hb];
            }
            V.template pv<PLO>(st + (kp % kStages) * G::STAGE, phi, plo, lane);
        }
        __syncthreads();
    }
    {
        // the last tile
        const int kp = ntl - 1;
        bf16x8 phi[4], plo[4];
        const lds_u8* pr = pm + (kp & 1) * PPAR + lane * 16;
        float al[4];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
            phi[hb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const lds_u32x4*>(pr + hb * 1024));
            if constexpr (PLO)
                plo[hb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const lds_u32x4*>(pr + 4096 + hb * 1024));
            al[hb] = alm[(kp & 1) * 64 + 16 * hb + c16];
        }
        if (__builtin_amdgcn_ballot_w64(al[0] != 1.0f || al[1] != 1.0f || al[2] != 1.0f || al[3] != 1.0f)) {
#pragma unroll
            for (int hb = 0; hb < 4; ++hb)
#pragma unroll
                for (int dt = 0; dt < VW::NDT; ++dt) V.o[hb][dt] *= al[hb];
        }
        V.template pv<PLO>(st + (kp % kStages) * G::STAGE, phi, plo, lane);
    }
    __syncthreads();                                         // matches the score waves' closing barrier
    __syncthreads();                                         // their m and l are in LDS
    // outputs of this quarter: lane (head c16 of block hb, g) holds dims
    // 16 dt + 4g .. +3
    constexpr int NDT = VW::NDT;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
        const int hl = 16 * hb + c16, hd = head0 + hl;
        const float l_tot = fin_mem[1][hl];
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        if (a.nsplit == 1) {
            const int64_t base = ((int64_t)r * a.H + hd) * DV + V.vbase + 4 * g;
            if (a.out_dtype == DT_F32) {
                float* out = reinterpret_cast<float*>(a.out) + base;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(out + 16 * dt) = V.o[hb][dt] * inv;
            } else {
                uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + base;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const f32x4 v = V.o[hb][dt] * inv;
                    *reinterpret_cast<u32x2*>(out + 16 * dt) = u32x2{cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3])};
                }
            }
        } else if (a.part_h) {
            // U = O / l, a convex combination of the values, as fp16 scaled by
            // 2^(15 - e) where max |U| over the lane's four dims < 2^e (no
            // cross-lane step; the scales are [row][split][tile][head][4]).
            // Partials are [row][split][16-dim tile][head][16 dims]: one store
            // writes 16 heads' tiles contiguously.
            const int64_t su = (int64_t)r * a.nsplit + split;
            uint16_t* ph = a.part_h + ((su * (DV / 16) + V.vbase / 16) * a.H + hd) * 16 + 4 * g;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                float amax = fmaxf(fmaxf(fabsf(V.o[hb][dt][0]), fabsf(V.o[hb][dt][1])),
                                   fmaxf(fabsf(V.o[hb][dt][2]), fabsf(V.o[hb][dt][3])));
                amax *= inv;
                int ex = 0;
                (void)frexpf(amax, &ex);
                const f32x4 v = V.o[hb][dt] * ldexpf(inv, 15 - ex);
                *reinterpret_cast<u32x2*>(ph + (int64_t)dt * a.H * 16) = u32x2{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
                a.part_sc[((su * (DV / 16) + V.vbase / 16 + dt) * a.H + hd) * 4 + g] = ldexpf(1.0f, ex - 15);
            }
        } else {
            const int64_t su = (int64_t)r * a.nsplit + split;
            float* po = a.part_o + ((su * (DV / 16) + V.vbase / 16) * a.H + hd) * 16 + 4 * g;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(po + (int64_t)dt * a.H * 16) = V.o[hb][dt];
        }
    }
}

// Merge the key splits of one (row, 16-dim tile of the values, 64 heads):
// per head m* = max m_s, w_s = 2^(m_s - m*), out = sum_s w_s O_s /
// sum_s w_s l_s, lse = (m* + log2 sum_s w_s l_s) ln 2.  With fp16 partials
// (HALF) a split stores U_s = O_s / l_s scaled by a power of two per 16 value
// dims, so its weight in the sum becomes w_s l_s times that scale.  Four
// threads per head, four value dims each; every thread forms its own head's
// weights from the (m, l) pairs, so the block needs no barrier.  Partials are
// [row][split][16-dim tile][head][16 dims] (scales [row][split][tile][head][4]),
// so a wave's load of one split reads 16 heads' tiles contiguously.  Splits
// are taken in chunks of MC whose loads are all issued at once (split indices
// past the last split re-read the last one and are masked; with at most 8
// splits the chunk is 8, which halves the registers a thread holds).  With
// more than 16 splits (MULTI) a workgroup covers 16 heads with four waves,
// wave g taking the chunks g, g + 4, ...: each folds its chunks with a
// running maximum, and wave 0 folds the other three's states from LDS.  Empty splits carry
// m = -inf, weight 0, and their workspace bytes are never used.
constexpr int kMergeThreads = 256;     // 64 heads x 4 threads
constexpr int kMergeChunk = 16;        // splits per chunk
constexpr int kMaxSplits = 256;

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

template <bool HALF, int MC, bool MULTI>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(AttnArgs a) {
    using MP = MergePart<HALF>;
    constexpr int NG = MULTI ? 4 : 1;                          // split groups (waves)
    const int tid = threadIdx.x, tile = blockIdx.x, r = blockIdx.y;
    const int grp = MULTI ? tid / 64 : 0;
    const int h = MULTI ? (int)blockIdx.z * 16 + (tid & 63) / 4 : (int)blockIdx.z * 64 + tid / 4;
    const int q = tid % 4;
    const int H = a.H, DV = a.d_v, ns = a.nsplit, NTL = DV / 16;
    const int64_t su0 = (int64_t)r * ns;
    const int64_t pstride = (int64_t)NTL * H * 16;            // partial values between splits
    const int64_t pbase = ((su0 * NTL + tile) * H + h) * 16 + 4 * q;
    const float2* ml = reinterpret_cast<const float2*>(a.part_ml) + su0 * H + h;   // (m, l) of split s at s * H
    const int64_t sstride = (int64_t)NTL * H * 4;             // scales between splits
    const float* scp = HALF ? a.part_sc + ((su0 * NTL + tile) * H + h) * 4 + q : nullptr;
    struct Chunk {
        typename MP::raw os[MC];
        float m[MC], l[MC], sc[HALF ? MC : 1];
    };
    auto load = [&](Chunk& c, int s0) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < MC; ++j) {
            const int64_t sj = min(s0 + j, ns - 1);
            c.os[j] = MP::load(a, pbase + sj * pstride);
            const float2 p = ml[sj * H];
            c.m[j] = p.x;
            c.l[j] = p.y;
            if constexpr (HALF) c.sc[j] = scp[sj * sstride];
        }
    };
    float M = -INFINITY, L = 0.0f;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    auto fold = [&](const Chunk& c, int s0) __attribute__((always_inline)) {
        float mc = -INFINITY;
#pragma unroll
        for (int j = 0; j < MC; ++j) mc = s0 + j < ns ? fmaxf(mc, c.m[j]) : mc;
        if (mc > M) {
            // a new running maximum: rescale what the earlier chunks summed
            const float f = __builtin_amdgcn_exp2f(M - mc);
            acc *= f;
            L *= f;
            M = mc;
        }
#pragma unroll
        for (int j = 0; j < MC; ++j) {
            const float w = s0 + j < ns && c.m[j] != -INFINITY ? __builtin_amdgcn_exp2f(c.m[j] - M) : 0.0f;
            L += w * c.l[j];
            const float ws = HALF ? w * c.l[j] * c.sc[HALF ? j : 0] : w;
            acc = w > 0.0f ? acc + ws * MP::value(c.os[j]) : acc;
        }
    };
    for (int s0 = grp * MC; s0 < ns; s0 += NG * MC) {
        Chunk c;
        load(c, s0);
        fold(c, s0);
    }
    if constexpr (MULTI) {
        // waves 1..3 hand (m, l, O) of their splits to wave 0
        __shared__ float xs[NG - 1][64][6];
        const int t = tid & 63;
        if (grp > 0) {
            float* x = xs[grp - 1][t];
            x[0] = M;
            x[1] = L;
#pragma unroll
            for (int i = 0; i < 4; ++i) x[2 + i] = acc[i];
        }
        __syncthreads();
        if (grp > 0) return;
#pragma unroll
        for (int g = 0; g < NG - 1; ++g) {
            const float* x = xs[g][t];
            const float mg = x[0];
            if (mg == -INFINITY) continue;
            if (mg > M) {
                const float f = __builtin_amdgcn_exp2f(M - mg);
                acc *= f;
                L *= f;
                M = mg;
            }
            const float f = __builtin_amdgcn_exp2f(mg - M);
            L += f * x[1];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += f * x[2 + i];
        }
    }
    if (a.lse && tile == 0 && q == 0) a.lse[(int64_t)r * H + h] = (M + log2f(L)) * kLn2;
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    acc *= inv;
    const int64_t oi = ((int64_t)r * H + h) * DV + tile * 16 + 4 * q;
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
    const int b = checked(a.row_seq[r], 0, a.batch - 1, a.dbg, kDbgRow);
    const int p = checked(a.row_pos[r], 0, a.max_pos, a.dbg, kDbgRow);
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
            const int pb = checked(a.block_table[(int64_t)b * a.max_blocks + g / E], 0, a.n_blocks - 1, a.dbg, kDbgBlock);
            return kvd + ((int64_t)pb * E + g % E) * D;
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
    if constexpr (KVD == DT_MXFP4) {
        if (a.q8) {
            if (a.p_lo) hipLaunchKernelGGL((attn_mfma_kernel<KVD, WD, D, DV, true, true>), grid, dim3(kThreads), 0, stream, a);
            else hipLaunchKernelGGL((attn_mfma_kernel<KVD, WD, D, DV, true, false>), grid, dim3(kThreads), 0, stream, a);
        } else {
            if (a.p_lo) hipLaunchKernelGGL((attn_mfma_kernel<KVD, WD, D, DV, false, true>), grid, dim3(kThreads), 0, stream, a);
            else hipLaunchKernelGGL((attn_mfma_kernel<KVD, WD, D, DV, false, false>), grid, dim3(kThreads), 0, stream, a);
        }
    } else {
        if (a.q8) return hipErrorInvalidValue;
        if (a.p_lo) hipLaunchKernelGGL((attn_mfma_kernel<KVD, WD, D, DV, false, true>), grid, dim3(kThreads), 0, stream, a);
        else hipLaunchKernelGGL((attn_mfma_kernel<KVD, WD, D, DV, false, false>), grid, dim3(kThreads), 0, stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    const dim3 mgrid(a.d_v / 16, a.num_rows, a.H / 64), mgrid16(a.d_v / 16, a.num_rows, a.H / 16);
    if (a.part_h) {
        if (a.nsplit <= kMergeChunk / 2) hipLaunchKernelGGL((attn_merge_kernel<true, kMergeChunk / 2, false>), mgrid, dim3(kMergeThreads), 0, stream, a);
        else if (a.nsplit <= kMergeChunk) hipLaunchKernelGGL((attn_merge_kernel<true, kMergeChunk, false>), mgrid, dim3(kMergeThreads), 0, stream, a);
        else hipLaunchKernelGGL((attn_merge_kernel<true, kMergeChunk, true>), mgrid16, dim3(kMergeThreads), 0, stream, a);
    } else {
        if (a.nsplit <= kMergeChunk / 2) hipLaunchKernelGGL((attn_merge_kernel<false, kMergeChunk / 2, false>), mgrid, dim3(kMergeThreads), 0, stream, a);
        else if (a.nsplit <= kMergeChunk) hipLaunchKernelGGL((attn_merge_kernel<false, kMergeChunk, false>), mgrid, dim3(kMergeThreads), 0, stream, a);
        else hipLaunchKernelGGL((attn_merge_kernel<false, kMergeChunk, true>), mgrid16, dim3(kMergeThreads), 0, stream, a);
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
int attn_max_split_tiles() { return kRowsLds / kKeys; }
int attn_max_splits() { return kMaxSplits; }
int attn_tile_keys() { return kKeys; }

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
