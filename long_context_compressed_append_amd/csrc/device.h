// Device helpers shared by the gfx950 kernels of liblcca: storage-format
// codecs (bf16, OCP E4M3, OCP MXFP4), wave reductions and MFMA operand types.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcca {

enum Dt : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2, DT_MXFP4 = 3, DT_NONE = -1 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
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

// E4M3 code -> bf16 bits (exact: 3 mantissa bits fit in bf16's 7).  Branch
// free: subnormal codes (exponent field 0) are m * 2^-9, formed in fp32.
__device__ inline uint32_t fp8_to_bf16(uint32_t c) {
    const uint32_t s = (c & 0x80u) << 8;
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    const uint32_t normal = ((e + 120u) << 7) | (m << 4);
    const uint32_t sub = __float_as_uint((float)m * 0.001953125f) >> 16;
    return s | (e == 0 ? sub : normal);
}

__device__ inline float fp8_to_f32(uint32_t c) { return bf16_to_f32(fp8_to_bf16(c)); }

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

// E2M1 code -> bf16 bits of code * 2^X.  The E2M1 magnitude (two significant
// bits) is formed in fp32, scaled by v_ldexp_f32 (exact for every E8M0 scale
// of fp32 data, subnormal results included) and truncated to bf16, which
// drops only zero bits.  Branch free.
__device__ inline uint32_t fp4_to_bf16(uint32_t nib, int X) {
    const uint32_t mag = nib & 7u;
    const uint32_t e = mag >> 1, mb = mag & 1u;
    uint32_t fb = ((126u + e) << 23) | (mb << 22);             // (1 + mb/2) * 2^(e-1), e >= 1
    fb = mag == 1u ? 0x3f000000u : fb;                         // 0.5
    fb = mag == 0u ? 0u : fb;
    const float v = ldexpf(__uint_as_float(fb), X);
    return ((nib & 8u) << 12) | (__float_as_uint(v) >> 16);
}

// Eight E4M3 codes (two words) -> eight bf16 (four words).
__device__ inline u32x4 fp8x8_to_bf16(uint32_t a, uint32_t b) {
    return u32x4{fp8_to_bf16(a & 0xffu) | (fp8_to_bf16((a >> 8) & 0xffu) << 16),
                 fp8_to_bf16((a >> 16) & 0xffu) | (fp8_to_bf16(a >> 24) << 16),
                 fp8_to_bf16(b & 0xffu) | (fp8_to_bf16((b >> 8) & 0xffu) << 16),
                 fp8_to_bf16((b >> 16) & 0xffu) | (fp8_to_bf16(b >> 24) << 16)};
}

// Eight E2M1 codes (one word, element 2i in the low nibble of byte i) with
// shared exponent X -> eight bf16 (four words).
__device__ inline u32x4 fp4x8_to_bf16(uint32_t w, int X) {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t bb = w >> (8 * q);
        o[q] = fp4_to_bf16(bb & 15u, X) | (fp4_to_bf16((bb >> 4) & 15u, X) << 16);
    }
    return o;
}

// ---------------------------------------------------------------------------
// wave helpers (wave64)
// ---------------------------------------------------------------------------
__device__ inline float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ inline float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ inline int visible_entries(int pos, int m) { return (pos + 1) / m; }

}  // namespace lcca
