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
// with one wave per 16 query heads.  Pipeline per workgroup:
//   prologue: the block-table range and the top-k indices the split needs are
//     copied to LDS, so resolving a key to its storage row is two LDS reads;
//   loads:    each tile's raw bytes (bf16, FP8 or MXFP4 + E8M0 scales) are
//     loaded into registers P tiles ahead of their use (static register sets,
//     loop unrolled by P), converted exactly to bf16 and written to one of two
//     padded LDS stages; one barrier per tile;
//   compute:  S^T = K Q^T with MFMA 16x16x32 (A = keys from LDS, B = the
//     wave's queries, resident in VGPRs); online softmax per lane in the exp2
//     domain; O^T += V^T P^T with V^T read from the same LDS tile by
//     ds_read_b64_tr_b16 (K = V); P enters as bf16 hi + lo so the value
//     weights keep 16 significant bits; FP8 window scales multiply the scores
//     and are folded into P.
// Keys are split across workgroups when the rows alone cannot fill the GPU;
// the partial (max, sum, unnormalised O) states go to the workspace and a
// merge kernel (one workgroup per row and head) combines them exactly.
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
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) int32_t lds_i32;

template <int N>
struct IntC {
    static constexpr int value = N;
};

template <int D>
struct Geo {
    static constexpr int ROWB = D * 2 + 16;          // padded bf16 row: conflict-free 16-B reads over 16 rows
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

    // Issue the loads of a resolved key into registers.
    __device__ __forceinline__ static void issue(const AttnArgs& a, const Src& s, TileRegs<NU>& R) {
        const int sub = (int)threadIdx.x % kThreadsPerKey;
        if (s.win) {
            const uint8_t* src = reinterpret_cast<const uint8_t*>(a.win_data) + s.row * (WD == DT_BF16 ? 2 * D : D);
#pragma unroll
            for (int i = 0; i < NU_W; ++i) {
                const int part = sub + kThreadsPerKey * i;
                const int pc = part < UPK_W ? part : 0;
                R.v[i] = *reinterpret_cast<const u32x4*>(src + pc * 16);
                R.sc[i] = 127u;
            }
            R.kscale = WD == DT_FP8 ? a.win_scale[s.row] : 1.0f;
        } else {
            const uint8_t* src = reinterpret_cast<const uint8_t*>(a.kv_data) + s.row * (KVD == DT_BF16 ? 2 * D : D / 2);
            const uint8_t* scs = reinterpret_cast<const uint8_t*>(a.kv_scale) + s.row * (D / 32);
#pragma unroll
            for (int i = 0; i < NU_P; ++i) {
                const int part = sub + kThreadsPerKey * i;
                const int pc = part < UPK_P ? part : 0;
                R.v[i] = *reinterpret_cast<const u32x4*>(src + pc * 16);
                R.sc[i] = KVD == DT_MXFP4 ? (uint32_t)scs[pc] : 127u;
            }
            R.kscale = 1.0f;
        }
        R.valid = s.ok;
    }

    // Convert the registers of tile `tile` to bf16 and write them to an LDS stage.
    // kmeta[0..31]: each key's value scale (FP8 window scale, 1, or -1 for
    // a masked key); kmeta[32..63]: its score factor scale_log2 * scale.
    __device__ __forceinline__ static void store(const RowKeys& rk, int tile, const TileRegs<NU>& R, lds_u8* stage,
                                                 lds_f32* kmeta, float scale_log2) {
        const int tid = threadIdx.x;
        const int key = tid / kThreadsPerKey, sub = tid % kThreadsPerKey;
        if (sub == 0) {
            kmeta[key] = R.valid ? R.kscale : -1.0f;
            kmeta[kKeys + key] = scale_log2 * R.kscale;
        }
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

// Per-wave softmax/PV state and the tile computation.  A pair of waves
// shares HB blocks of 16 heads and splits the shared-KV dimension: each wave
// computes the partial scores over its half of D (its half of every query
// stays in VGPRs), the pair swaps partial scores through LDS, and each wave
// then runs the same softmax and accumulates P V for its half of the value
// dims.  Every key or value fragment read from LDS feeds HB head blocks.
template <int D, int DV, int HB>
struct HalfWave {
    static constexpr int KS = D / 64;          // k-steps of S^T per half
    static constexpr int NDT = DV / 32;        // 16-dim tiles of O^T per half
    static constexpr int NACC = HB == 1 ? 2 : 1;   // accumulators per score sub-tile
    static constexpr int XS = HB * 8 * 64;     // floats of one wave's score exchange slot
    bf16x8 qb[HB][KS];
    f32x4 o[HB][NDT];
    float m_run[HB], l_run[HB];

    __device__ __forceinline__ void init(const AttnArgs& a, int r, int head0, int g, int half) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const uint16_t* q =
                reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)r * a.H + head0 + 16 * hb) * D + half * (D / 2);
#pragma unroll
            for (int s = 0; s < KS; ++s)
                qb[hb][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q + 32 * s + 8 * g));
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) o[hb][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            m_run[hb] = -INFINITY;
            l_run[hb] = 0.0f;
        }
    }

    // xs_mine / xs_pair: this wave's and the partner wave's score exchange
    // slots, [HB][64 lanes][8] floats each.
    __device__ __forceinline__ void tile(const lds_u8* lds, const lds_f32* kmeta, lds_f32* xs_mine,
                                         const lds_f32* xs_pair, int g, int c16, int lane, int half) {
        constexpr int ROWB = Geo<D>::ROWB;
        // partial S^T = K Q^T over this half's dims: two 16-key sub-tiles per
        // head block; each key fragment serves every head block
        f32x4 sacc[2][HB][NACC];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
#pragma unroll
                for (int c = 0; c < NACC; ++c) sacc[kt][hb][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            bf16x8 kA[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                kA[kt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const lds_u32x4*>(
                                                        lds + (kt * 16 + c16) * ROWB + half * D + 16 * g + 64 * s));
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int hb = 0; hb < HB; ++hb)
                    sacc[kt][hb][s % NACC] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA[kt], qb[hb][s], sacc[kt][hb][s % NACC], 0, 0, 0);
        }
        f32x4 sp[2][HB];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
                sp[kt][hb] = sacc[kt][hb][0];
                if constexpr (NACC > 1) sp[kt][hb] += sacc[kt][hb][1];
                *reinterpret_cast<lds_f32x4*>(xs_mine + (hb * 64 + lane) * 8 + 4 * kt) = sp[kt][hb];
            }
        __syncthreads();
        bf16x8 pb[HB], pbl[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            float x[2][4], ks[2][4];
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const f32x4 pair = *reinterpret_cast<const lds_f32x4*>(xs_pair + (hb * 64 + lane) * 8 + 4 * kt);
                const f32x4 km = *reinterpret_cast<const lds_f32x4*>(kmeta + kt * 16 + 4 * g);
                const f32x4 kx = *reinterpret_cast<const lds_f32x4*>(kmeta + kKeys + kt * 16 + 4 * g);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    ks[kt][v] = km[v];
                    x[kt][v] = km[v] >= 0.0f ? (sp[kt][hb][v] + pair[v]) * kx[v] : -INFINITY;
                    mx = fmaxf(mx, x[kt][v]);
                }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            // Lazy rescaling: the reference max m_run moves only when the tile's
            // max exceeds it by more than 8 (log2 units), so most tiles leave the
            // O accumulators untouched; probabilities relative to m_run stay <= 2^8.
            if (mx > m_run[hb] + 8.0f) {
                const float alpha = exp2f(m_run[hb] - mx);     // 0 while m_run = -inf
                l_run[hb] *= alpha;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) o[hb][dt] *= alpha;
                m_run[hb] = mx;
            }
            // reference for the exponent: m_run, or 0 while every key so far is
            // masked (then every x is -inf and every p is 0)
            const float mref = m_run[hb] == -INFINITY ? 0.0f : m_run[hb];
            float psum = 0.0f;
            uint32_t pk[4], pl[4];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int v = 0; v < 4; v += 2) {
                    // x - mref <= 8: v_exp_f32 directly (results below 2^-126
                    // may flush to zero, far below the sum's precision)
                    const float p0 = __builtin_amdgcn_exp2f(x[kt][v] - mref);
                    const float p1 = __builtin_amdgcn_exp2f(x[kt][v + 1] - mref);
                    psum += p0 + p1;
                    // masked keys have p = 0; FP8 window keys carry their scale
                    const float w0 = p0 * ks[kt][v], w1 = p1 * ks[kt][v + 1];
                    const uint32_t h = cvt_pk_bf16(w0, w1);
                    pk[kt * 2 + v / 2] = h;
                    pl[kt * 2 + v / 2] = cvt_pk_bf16(w0 - __uint_as_float(h << 16), w1 - __uint_as_float(h & 0xffff0000u));
                }
            l_run[hb] += psum;
            pb[hb] = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
            pbl[hb] = __builtin_bit_cast(bf16x8, u32x4{pl[0], pl[1], pl[2], pl[3]});
        }
        // O^T += V^T P^T over this half's value dims.  Within each 16-lane block,
        // ds_read_b64_tr_b16 hands lane i element (i & 3) of the 8-byte chunk
        // addressed by lane (i >> 2) + 4e, e = 0..3: lane s addresses key
        // 4g + (s >> 2), dims dt*16 + 4(s & 3) .. +3, so lane i receives keys
        // 4g + e at dim dt*16 + i.  Each value fragment serves every head
        // block, hi and lo; the hi and lo products of a dim tile are issued
        // apart so they do not wait on each other.
        const lds_u8* vbase = lds + (4 * g + (c16 >> 2)) * ROWB + half * (DV / 2) * 2 + 8 * (c16 & 3);
        constexpr int G4 = HB == 1 ? 4 : 2;
#pragma unroll
        for (int d0 = 0; d0 < NDT; d0 += G4) {
            bf16x8 vA[G4];
#pragma unroll
            for (int j = 0; j < G4; ++j) {
                if (d0 + j < NDT) {
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
                for (int hb = 0; hb < HB; ++hb)
                    if (d0 + j < NDT)
                        o[hb][d0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA[j], pb[hb], o[hb][d0 + j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < G4; ++j)
#pragma unroll
                for (int hb = 0; hb < HB; ++hb)
                    if (d0 + j < NDT)
                        o[hb][d0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA[j], pbl[hb], o[hb][d0 + j], 0, 0, 0);
        }
    }
};

constexpr int kHeadBlocks = 1;         // 16-head blocks per wave
constexpr int kBtLds = 4096;           // block-table entries cached in LDS
constexpr int kIdxLds = 2560;          // top-k slots cached in LDS (= max keys per split)

template <int KVD, int WD, int D, int DV, int HB>
__global__ __launch_bounds__(8 / HB * 64) __attribute__((amdgpu_waves_per_eu(2 / HB, 2 / HB))) void attn_mfma_kernel(
    AttnArgs a) {
    constexpr int NW = 8 / HB;                                    // waves: NW/2 head groups x 2 halves of D
    using G = Geo<D>;
    constexpr int NT = NW * 64;
    using TL = Tiler<KVD, WD, D, NT>;
    constexpr int NU = TL::NU;
    // tiles held in registers ahead of the LDS stage
    constexpr int kPrefetch = NU <= 12 ? 2 : 1;
    static_assert(kPrefetch == 1 || kPrefetch == 2, "prefetch depth");
    __shared__ __attribute__((aligned(16))) uint8_t stage[2][G::STAGE];
    __shared__ __attribute__((aligned(16))) float kmeta[2][2 * kKeys];
    __shared__ int32_t bt_mem[kBtLds];
    __shared__ int32_t idx_mem[kIdxLds];
    __shared__ __attribute__((aligned(16))) float xs_mem[NW][HalfWave<D, DV, HB>::XS];   // partial-score exchange
    lds_i32* const bt_lds = (lds_i32*)&bt_mem[0];
    lds_i32* const idx_lds = (lds_i32*)&idx_mem[0];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int split = blockIdx.x, r = blockIdx.y;
    const RowKeys rk = row_keys(a, r);
    const int tb = split * a.split_tiles;
    if (tb >= rk.tiles) {
        // empty split (a row with fewer tiles than the longest): a zero state
        if (a.nsplit > 1 && tid < 64) {
            float* ml = a.part_ml + ((int64_t)r * a.nsplit + split) * 2 * a.H + (int)blockIdx.z * 64 + tid;
            ml[0] = -INFINITY;
            ml[a.H] = 0.0f;
        }
        return;
    }
    const int te = min(tb + a.split_tiles, rk.tiles);
    // waves w and w + NW/2 share 16 HB heads and split the dimensions
    const int hg = wave % (NW / 2), half = wave / (NW / 2);
    const int head = (int)blockIdx.z * 64 + hg * 16 * HB + c16;   // this lane's head of head block 0

    // prologue: top-k slots and block-table range of this split into LDS
    const int sel_end = min(te, rk.sel_tiles) * kKeys;            // selected slots [tb*32, sel_end)
    const int idx0 = tb * kKeys;
    int blk0 = 0, nblk = 0;
    if (sel_end > idx0) {
        const int E = 256 / a.m;
        if (a.topk) {
            nblk = (rk.n + E - 1) / E;
            for (int i = tid; i < sel_end - idx0; i += NT)
                idx_lds[i] = idx0 + i < rk.nsel ? a.topk[(int64_t)r * a.k + idx0 + i] : -1;
        } else {
            const int g1 = min(sel_end, rk.nsel);
            if (g1 > idx0) {
                blk0 = idx0 / E;
                nblk = (g1 - 1) / E - blk0 + 1;
            }
        }
    }
    for (int i = tid; i < min(nblk, kBtLds); i += NT) bt_lds[i] = a.block_table[(int64_t)rk.b * a.max_blocks + blk0 + i];
    __syncthreads();

    HalfWave<D, DV, HB> W;
    W.init(a, r, head, g, half);
    lds_f32* const xs_mine = (lds_f32*)&xs_mem[wave][0];
    const lds_f32* const xs_pair = (lds_f32*)&xs_mem[wave ^ (NW / 2)][0];

    TileRegs<NU> R[kPrefetch];
    const int ntl = te - tb;
    TL::issue(a, TL::resolve(a, rk, tb, true, idx_lds, idx0, bt_lds, blk0), R[0]);
    if constexpr (kPrefetch > 1) TL::issue(a, TL::resolve(a, rk, tb + 1, 1 < ntl, idx_lds, idx0, bt_lds, blk0), R[1]);
    lds_u8* const st = (lds_u8*)&stage[0][0];
    lds_f32* const km = (lds_f32*)&kmeta[0][0];
    TL::store(rk, tb, R[0], st, km, a.scale_log2);
    TL::issue(a, TL::resolve(a, rk, tb + kPrefetch, kPrefetch < ntl, idx_lds, idx0, bt_lds, blk0), R[0]);
    __syncthreads();

    // tile u sits in register set (u - tb) % P until it is stored to stage
    // (u - tb) % 2; the steps of one round are spelled out so that every
    // register set is addressed statically
    auto step = [&](auto J, int t) __attribute__((always_inline)) {
        constexpr int nxt = (decltype(J)::value + 1) % kPrefetch;
        // the next loads' storage rows come from LDS before this step's stores
        const typename TL::Src nsrc =
            TL::resolve(a, rk, tb + t + 1 + kPrefetch, t + 1 + kPrefetch < ntl, idx_lds, idx0, bt_lds, blk0);
        if (t + 1 < ntl)
            TL::store(rk, tb + t + 1, R[nxt], st + ((t + 1) & 1) * G::STAGE, km + ((t + 1) & 1) * 2 * kKeys, a.scale_log2);
        TL::issue(a, nsrc, R[nxt]);
        W.tile(st + (t & 1) * G::STAGE, km + (t & 1) * 2 * kKeys, xs_mine, xs_pair, g, c16, lane, half);
        __syncthreads();
    };
    for (int t0 = 0; t0 < ntl; t0 += kPrefetch) {
        step(IntC<0>{}, t0);
        if constexpr (kPrefetch > 1)
            if (t0 + 1 < ntl) step(IntC<1>{}, t0 + 1);
    }

    // finish: total row sum of each head over the 4 lane groups
    constexpr int NDT = HalfWave<D, DV, HB>::NDT;
    const int dv0 = half * (DV / 2) + 4 * g;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        const int hd = head + 16 * hb;
        float l_tot = W.l_run[hb] + __shfl_xor(W.l_run[hb], 16);
        l_tot += __shfl_xor(l_tot, 32);
        if (a.nsplit == 1) {
            const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            const int64_t base = ((int64_t)r * a.H + hd) * DV + dv0;
            if (a.out_dtype == DT_F32) {
                float* out = reinterpret_cast<float*>(a.out) + base;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(out + dt * 16) = W.o[hb][dt] * inv;
            } else {
                uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + base;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    f32x4 t = W.o[hb][dt] * inv;
                    *reinterpret_cast<u32x2*>(out + dt * 16) = u32x2{cvt_pk_bf16(t[0], t[1]), cvt_pk_bf16(t[2], t[3])};
                }
            }
            if (a.lse && g == 0 && half == 0) a.lse[(int64_t)r * a.H + hd] = (W.m_run[hb] + log2f(l_tot)) * kLn2;
        } else {
            float* po = a.part_o + (((int64_t)r * a.nsplit + split) * a.H + hd) * DV + dv0;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = W.o[hb][dt];
            if (g == 0 && half == 0) {
                float* ml = a.part_ml + ((int64_t)r * a.nsplit + split) * 2 * a.H;
                ml[hd] = W.m_run[hb];
                ml[a.H + hd] = l_tot;
            }
        }
    }
}

// Merge the key splits of one (row, head): m* = max m_s, w_s = 2^(m_s - m*),
// out = sum_s w_s O_s / sum_s w_s l_s, lse = (m* + log2 sum_s w_s l_s) ln 2.
// Each thread owns 4 value dims.  The partial outputs of the first
// kMergeBatch splits are requested before anything else, so they are in
// flight while the block forms the weights (thread s owns split s and
// s + kMergeThreads).  Empty splits carry m = -inf, weight 0, and their
// workspace bytes are never used.
constexpr int kMergeThreads = 192;     // >= 576 / 4
constexpr int kMaxSplits = 256;        // <= 2 * kMergeThreads
constexpr int kMergeBatch = 16;
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(AttnArgs a) {
    __shared__ float wts[kMaxSplits];
    __shared__ float red[2][kMergeThreads / 64];
    const int h = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
    const int H = a.H, DV = a.d_v, ns = a.nsplit;
    const float* ml = a.part_ml + (int64_t)r * ns * 2 * H + h;
    const int d = 4 * tid;
    const bool mine = d < DV;
    const float* po = a.part_o + ((int64_t)r * ns * H + h) * DV + (mine ? d : 0);
    const int64_t sstride = (int64_t)H * DV;
    f32x4 os[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) os[j] = *reinterpret_cast<const f32x4*>(po + min(j, ns - 1) * sstride);
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
    if (tid < ns) wts[tid] = w0;
    if (s1 < ns) wts[s1] = w1;
    float L = wave_sum(w0 * l0 + w1 * l1);
    if ((tid & 63) == 0) red[1][tid >> 6] = L;
    __syncthreads();
    L = 0.0f;
#pragma unroll
    for (int i = 0; i < kMergeThreads / 64; ++i) L += red[1][i];
    if (a.lse && tid == 0) a.lse[(int64_t)r * H + h] = (M + log2f(L)) * kLn2;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
        const float w = j < ns ? wts[j] : 0.0f;
        acc = w > 0.0f ? acc + w * os[j] : acc;
    }
    for (int s0 = kMergeBatch; s0 < ns; s0 += kMergeBatch) {
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) os[j] = *reinterpret_cast<const f32x4*>(po + min(s0 + j, ns - 1) * sstride);
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
            const float w = s0 + j < ns ? wts[s0 + j] : 0.0f;
            acc = w > 0.0f ? acc + w * os[j] : acc;
        }
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

template <int KVD, int WD, int D, int DV, int HB>
hipError_t launch_mfma(const AttnArgs& a, hipStream_t stream) {
    dim3 grid(a.nsplit, a.num_rows, a.H / 64);
    hipLaunchKernelGGL((attn_mfma_kernel<KVD, WD, D, DV, HB>), grid, dim3(8 / HB * 64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(a.H, a.num_rows), dim3(kMergeThreads), 0, stream, a);
    return hipGetLastError();
}

// Workgroups cover 64 heads (eight waves of 16 heads each); more heads add
// head groups to the grid.
template <int KVD, int WD, int D, int DV>
hipError_t launch_heads(const AttnArgs& a, hipStream_t stream) {
    if (a.H % 64 != 0) return hipErrorInvalidValue;
    return launch_mfma<KVD, WD, D, DV, kHeadBlocks>(a, stream);
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
