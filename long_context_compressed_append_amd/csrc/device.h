// Device helpers shared by the gfx950 kernels of liblcca: storage-format
// codecs (bf16, OCP E4M3, OCP MXFP4), wave reductions and MFMA operand types.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcca {

enum Dt : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2, DT_MXFP4 = 3, DT_NONE = -1 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__host__ __device__ inline int64_t row_bytes(int dtype, int dim) {
    return dtype == DT_F32 ? 4LL * dim : dtype == DT_BF16 ? 2LL * dim : dtype == DT_FP8 ? (int64_t)dim : dim / 2;
}

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------
__device__ inline float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN).
__device__ inline uint32_t f32_to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) { return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// The same rounding in one instruction (v_cvt_pk_bf16_f32, round to nearest
// even) for finite values: attention probabilities and outputs.
// fp16 (IEEE binary16), round to nearest even, two per word (low first).
__device__ inline uint32_t pack_f16x2(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}
__device__ inline float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ inline float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

__device__ inline uint32_t cvt_pk_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// ---------------------------------------------------------------------------
// OCP E4M3 ("fn": bias 7, max 448, S.1111.111 = NaN)
// ---------------------------------------------------------------------------

// fp32 -> E4M3, round to nearest even, saturating to +-448.
__device__ inline uint32_t f32_to_fp8(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t ua = u & 0x7fffffffu;
    if (ua > 0x7f800000u) return sign | 0x7fu;                 // NaN
    float a = __uint_as_float(ua);
    if (a >= 448.0f) return sign | 0x7eu;
    if (a < 0.015625f) {                                       // below 2^-6: multiples of 2^-9
        float q = rintf(a * 512.0f);                           // exact scaling, RNE
        return sign | (uint32_t)q;                             // q == 8 encodes 2^-6 (e=1, m=0)
    }
    uint32_t r = ua + 0x7ffffu + ((ua >> 20) & 1u);            // RNE to 3 mantissa bits
    int e = (int)(r >> 23) - 127;
    uint32_t m3 = (r >> 20) & 7u;
    if (e > 8 || (e == 8 && m3 == 7u)) return sign | 0x7eu;    // rounded past 448
    return sign | ((uint32_t)(e + 7) << 3) | m3;
}

// The same rounding for finite |x| < 448 without branches (both encodings
// are formed and one is selected), for code paths where lanes hold values
// of every binade.
__device__ __forceinline__ uint32_t f32_to_fp8_inrange(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t ua = u & 0x7fffffffu;
    const float a = __uint_as_float(ua);
    const uint32_t sub = (uint32_t)rintf(a * 512.0f);                   // below 2^-6: multiples of 2^-9
    const uint32_t r = ua + 0x7ffffu + ((ua >> 20) & 1u);               // RNE to 3 mantissa bits
    const uint32_t nor = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);  // (e + 7) << 3 | m3
    return sign | (a < 0.015625f ? sub : nor);
}

// E4M3 code -> value (finite codes), without branches.
__device__ __forceinline__ float fp8_value(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    const float sub = (float)m * 0x1p-9f;
    const float nor = ldexpf(1.0f + (float)m * 0.125f, (int)e - 7);
    const float v = e == 0 ? sub : nor;
    return (c & 0x80u) ? -v : v;
}

// ---------------------------------------------------------------------------
// OCP MXFP4: E2M1 elements, one E8M0 scale per 32 elements
// ---------------------------------------------------------------------------

// |v| -> E2M1 magnitude code (v already divided by 2^X), nearest, ties to
// the even mantissa, saturating at 6.
__device__ inline uint32_t fp4_code(float v) {
    uint32_t sign = (__float_as_uint(v) >> 28) & 8u;
    float a = fabsf(v);
    uint32_t c;
    if (a <= 0.25f) c = 0;
    else if (a < 0.75f) c = 1;
    else if (a <= 1.25f) c = 2;
    else if (a < 1.75f) c = 3;
    else if (a <= 2.5f) c = 4;
    else if (a < 3.5f) c = 5;
    else if (a <= 5.0f) c = 6;
    else c = 7;                                                // also NaN -> saturate
    return sign | c;
}

// Shared exponent X = floor(log2(amax)) - 2, clamped to [-127, 127].
__device__ inline int mx_scale_exp(float amax) {
    if (!(amax > 0.0f)) return -127;
    int ex;
    frexpf(amax, &ex);
    int X = ex - 1 - 2;
    return X < -127 ? -127 : (X > 127 ? 127 : X);
}

// Decoding uses gfx950's scaled conversions (v_cvt_scalef32_pk_bf16_fp8 /
// _fp4: two OCP codes -> two bf16, times a float scale).  Every E4M3 value
// and every E2M1 value times a power-of-two scale 2^X, X >= -126, is a bf16
// value, so the conversion is exact; for X = -127 (the scale of an all-zero
// block, or of a block below 2^-125) the scale operand 2^-127 is a float
// subnormal and the block decodes to zeros, an absolute error below 2^-124.

// Eight E4M3 codes (two words, code i in byte i) -> eight bf16 (four words).
__device__ inline u32x4 fp8x8_to_bf16(uint32_t a, uint32_t b) {
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a, 1.0f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b, 1.0f, true))};
}

// Eight E2M1 codes (one word, element 2i in the low nibble of byte i) with
// shared exponent X -> eight bf16 (four words).
__device__ inline u32x4 fp4x8_to_bf16(uint32_t w, int X) {
    const float sc = __uint_as_float(X > -127 ? (uint32_t)(X + 127) << 23 : 0u);
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3))};
}

// ---------------------------------------------------------------------------
// wave helpers (wave64)
// ---------------------------------------------------------------------------
// v of lane l ^ O, on the VALU: quad permutations (O = 1, 2), row shifts
// within 16-lane rows selected by lane bit 2 (O = 4: lane l reads l + 4 or
// l - 4), a rotation of each row by 8 (O = 8), and the permlane swaps across
// rows and wave halves (O = 16, 32; their two results hold lane l's and its
// partner's values, in an order set by lane bit 4 or 5).  No LDS round trip.
template <int O>
__device__ __forceinline__ float lane_xor(float v) {
    const int x = __float_as_int(v);
    const int lane = (int)threadIdx.x & 63;
    if constexpr (O == 1) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
    } else if constexpr (O == 2) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
    } else if constexpr (O == 4) {
        const int up = __builtin_amdgcn_update_dpp(0, x, 0x104, 0xF, 0xF, false);          // row_shl:4
        const int dn = __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);          // row_shr:4
        return __int_as_float((lane & 4) ? dn : up);
    } else if constexpr (O == 8) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false));   // row_ror:8
    } else if constexpr (O == 16) {
        const auto a = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
        return __uint_as_float((lane & 16) ? a[0] : a[1]);
    } else {
        static_assert(O == 32, "lane_xor: O is a power of two up to 32");
        const auto a = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
        return __uint_as_float((lane & 32) ? a[0] : a[1]);
    }
}

// Butterfly reductions over the wave (every lane gets the result), pairing
// lanes l and l ^ o for o = 32, 16, ..., 1: each lane adds its own value and
// its partner's, so every lane holds the same bits.
__device__ inline float wave_max(float v) {
    v = fmaxf(v, lane_xor<32>(v));
    v = fmaxf(v, lane_xor<16>(v));
    v = fmaxf(v, lane_xor<8>(v));
    v = fmaxf(v, lane_xor<4>(v));
    v = fmaxf(v, lane_xor<2>(v));
    return fmaxf(v, lane_xor<1>(v));
}
__device__ inline float wave_sum(float v) {
    v += lane_xor<32>(v);
    v += lane_xor<16>(v);
    v += lane_xor<8>(v);
    v += lane_xor<4>(v);
    v += lane_xor<2>(v);
    return v + lane_xor<1>(v);
}

// max of v over lanes l, l ^ 16, l ^ 32 and l ^ 48, on the VALU (gfx950's
// v_permlane32_swap exchanges the upper 32 lanes of one operand with the
// lower 32 of the other, v_permlane16_swap the odd 16-lane rows of one with
// the even rows of the other; with both operands holding v, the two results
// hold the two partners' values, in some order).
__device__ inline float max_across_rows(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// v of lane l plus v of lane l ^ 32, on the VALU (as above; the sum of the
// two is the same whichever result holds which).
__device__ inline float sum_halves(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

__device__ inline int visible_entries(int pos, int m) { return (pos + 1) / m; }

// ---------------------------------------------------------------------------
// Index checks of the debug build
// ---------------------------------------------------------------------------
// With LCCA_DEBUG defined, an index read from device memory is tested against
// its range [lo, hi] before it forms an address; outside it, `lo` is used
// instead and `bit` is set in the device error word `word`, so every load
// stays inside its buffer and the kernel finishes normally.  Without
// LCCA_DEBUG the value is used as read (the caller vouches for it).
__device__ __forceinline__ int checked(int v, int lo, int hi, uint32_t* word, uint32_t bit) {
#ifdef LCCA_DEBUG
    if (v < lo || v > hi) {
        atomicOr(word, bit);
        return lo;
    }
#endif
    (void)lo; (void)hi; (void)word; (void)bit;
    return v;
}

// Whether a debug build has found a chunk description invalid (cu_new and
// start_pos of new token t, as read): always false in release builds.
__device__ __forceinline__ bool chunk_invalid(int t, int c0, int c1, int start, int total_new, int max_blocks,
                                              uint32_t* word, uint32_t bit) {
#ifdef LCCA_DEBUG
    const bool bad = c0 < 0 || c0 > t || c1 <= t || c1 > total_new || start < 0 ||
                     (int64_t)start + (c1 - c0) > (int64_t)max_blocks * 256;
    if (bad) atomicOr(word, bit);
    return bad;
#else
    (void)t; (void)c0; (void)c1; (void)start; (void)total_new; (void)max_blocks; (void)word; (void)bit;
    return false;
#endif
}

// Order-preserving u32 key of a logit (-0.0 folded onto +0.0): larger
// logits have larger keys.  The top-k selection ranks by it, and the
// decode indexer counts the leading kTopkLeadBits bits of its logits' keys
// with it.
__device__ inline uint32_t order_key(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;                               // -0.0 ties +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace lcca
