// sparse_attn_fwd: single-KV-head attention of H query heads over the
// selected compressed entries plus the sliding window, one joint softmax.
//
// [P1 = page "vLLM uveo DeepSeek V4 s 8,7x manjim KV cacheom", section
//  "Kako funkcionira optimizacija KV cachea?": shared KV vectors (one vector
//  is key and value), attention restricted to the top-k compressed tokens,
//  and a local window of full vectors for recent context.  P3 = page
//  "DeepSeek-V4.1-Flash ve vLLM: kde se vzala 5,3x vyssi propustnost",
//  section "Vykon neprinesl jeden kernel": the fused attention reads a 4-bit
//  compressed cache; here MXFP4 (OCP) or bf16 entries and an FP8 or bf16
//  window are dequantised while staging into LDS.]
//
// bf16/MFMA path.  A workgroup = (row, key split) with one wave per 16 query
// heads.  Per 32-key tile:
//   1. the workgroup gathers the tile (block table / window ring), converts
//      it exactly to bf16 and stages it in LDS ([32][D] + pad);
//   2. each wave computes S^T = K Q^T with MFMA 16x16x32 (A = keys from LDS,
//      B = its heads' queries, resident in VGPRs), so every lane owns one
//      head and 8 keys;
//   3. online softmax in the exp2 domain, entirely per lane plus two
//      cross-lane max/sum steps; FP8 window scales multiply the scores and
//      are folded into P for the value product;
//   4. O^T += V^T P^T with MFMA 16x16x32: the P operand is the softmax
//      result already in the right registers, V^T is read from the same LDS
//      tile (K = V) transposed; O^T stays in registers with one head per
//      lane, so the softmax rescale is a per-lane multiply.
// Keys are split across workgroups when there are too few rows to fill the
// GPU; partial (max, sum, unnormalised O) states go to the workspace and a
// merge kernel combines them exactly.
#include "device.h"
#include "kernels.h"

namespace lcca {

namespace {

constexpr float kLn2 = 0.69314718055994530942f;

template <int D>
struct Tile {
    static constexpr int ROWB = D * 2 + 16;          // padded row: conflict-free 16-B reads across 16 rows
    static constexpr int KEYS = 32;
    static constexpr int CPK = D / 8;                // 16-byte bf16 chunks per key
};

// Key list of a row: [selected entries (k slots, or every visible entry)] ++
// [window tokens max(0, p-window+1) .. p].
struct RowKeys {
    int b, p, n, nsel, t0, L;
};

__device__ inline RowKeys row_keys(const AttnArgs& a, int r) {
    RowKeys k;
    k.b = a.row_seq[r];
    k.p = a.row_pos[r];
    k.n = visible_entries(k.p, a.m);
    k.nsel = a.topk ? a.k : k.n;
    k.t0 = max(0, k.p - a.window + 1);
    k.L = k.nsel + (k.p - k.t0 + 1);
    return k;
}

// Resolve list position j to a storage row.  kind: 0 = invalid, 1 = pool
// entry (row in the pool), 2 = window slot (row = b*cap + t % cap).
__device__ inline void resolve_key(const AttnArgs& a, const RowKeys& rk, int r, int j, int j_end, int& kind,
                                   int64_t& row) {
    kind = 0;
    row = 0;
    if (j >= j_end) return;
    if (j < rk.nsel) {
        int g = a.topk ? a.topk[(int64_t)r * a.k + j] : j;
        if (g < 0 || g >= rk.n) return;
        const int E = 256 / a.m;
        row = (int64_t)a.block_table[(int64_t)rk.b * a.max_blocks + g / E] * E + g % E;
        kind = 1;
    } else {
        int t = rk.t0 + (j - rk.nsel);
        row = (int64_t)rk.b * a.win_cap + t % a.win_cap;
        kind = 2;
    }
}

template <int KVD, int WD, int D, int DV, int NW>
__global__ __launch_bounds__(NW * 64) void attn_mfma_kernel(AttnArgs a) {
    using T = Tile<D>;
    constexpr int NT = NW * 64;
    constexpr int KS = D / 32;          // k-steps of S^T
    constexpr int NDT = DV / 16;        // 16-dim tiles of O^T
    __shared__ __attribute__((aligned(16))) uint8_t lds[T::KEYS * T::ROWB];
    __shared__ int64_t src_row[T::KEYS];
    __shared__ int src_kind[T::KEYS];
    __shared__ float kscale[T::KEYS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int split = blockIdx.x, r = blockIdx.y;
    const RowKeys rk = row_keys(a, r);
    const int j_begin = split * a.split_keys;
    if (j_begin >= rk.L) return;                                  // empty split (merge skips it)
    const int j_end = min(j_begin + a.split_keys, rk.L);
    const int head = wave * 16 + c16;

    // Q^T as B operands: lane (head, g) holds dims [32s + 8g, +8)
    bf16x8 qb[KS];
    {
        const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)r * a.H + head) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) qb[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q + 32 * s + 8 * g));
    }
    f32x4 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    const uint8_t* kvd = reinterpret_cast<const uint8_t*>(a.kv_data);
    const uint8_t* kvs = reinterpret_cast<const uint8_t*>(a.kv_scale);
    const uint8_t* wdat = reinterpret_cast<const uint8_t*>(a.win_data);

    for (int j0 = j_begin; j0 < j_end; j0 += T::KEYS) {
        // 1a. resolve the tile's keys
        if (tid < T::KEYS) {
            int kind; int64_t row;
            resolve_key(a, rk, r, j0 + tid, j_end, kind, row);
            src_row[tid] = row;
            src_kind[tid] = kind;
            kscale[tid] = (kind == 2 && WD == DT_FP8) ? a.win_scale[row] : 1.0f;
        }
        __syncthreads();
        // 1b. gather + dequantise into LDS (16-byte bf16 chunks)
        for (int c = tid; c < T::KEYS * T::CPK; c += NT) {
            const int kk = c / T::CPK, part = c - kk * T::CPK;
            const int kind = src_kind[kk];
            const int64_t row = src_row[kk];
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (kind == 1) {
                if (KVD == DT_BF16) {
                    v = *reinterpret_cast<const u32x4*>(kvd + row * (2 * D) + part * 16);
                } else {   // MXFP4: 8 nibbles + the block's E8M0 scale
                    uint32_t w = *reinterpret_cast<const uint32_t*>(kvd + row * (D / 2) + part * 4);
                    int X = (int)kvs[row * (D / 32) + part / 4] - 127;
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        uint32_t bb = w >> (8 * h);
                        v[h] = fp4_to_bf16(bb & 15u, X) | (fp4_to_bf16((bb >> 4) & 15u, X) << 16);
                    }
                }
            } else if (kind == 2) {
                if (WD == DT_BF16) {
                    v = *reinterpret_cast<const u32x4*>(wdat + row * (2 * D) + part * 16);
                } else {   // FP8 codes; the per-token scale is applied to scores and P
                    u32x2 w = *reinterpret_cast<const u32x2*>(wdat + row * D + part * 8);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        uint32_t x = w[h];
                        v[2 * h] = fp8_to_bf16(x & 0xffu) | (fp8_to_bf16((x >> 8) & 0xffu) << 16);
                        v[2 * h + 1] = fp8_to_bf16((x >> 16) & 0xffu) | (fp8_to_bf16(x >> 24) << 16);
                    }
                }
            }
            *reinterpret_cast<u32x4*>(lds + kk * T::ROWB + part * 16) = v;
        }
        __syncthreads();

        // 2. S^T = K Q^T: two 16-key sub-tiles
        f32x4 sacc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const uint8_t* rowp = lds + (kt * 16 + c16) * T::ROWB + 16 * g;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                bf16x8 kA = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(rowp + 64 * s));
                sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA, qb[s], sacc[kt], 0, 0, 0);
            }
        }
        // 3. online softmax (log2 domain); lane holds keys kt*16 + 4g + v of head `head`
        float x[2][4];
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int kk = kt * 16 + 4 * g + v;
                float sc = sacc[kt][v] * a.scale_log2 * kscale[kk];
                x[kt][v] = src_kind[kk] ? sc : -INFINITY;
                mx = fmaxf(mx, x[kt][v]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const bool none = m_new == -INFINITY;
        const float alpha = none ? 1.0f : exp2f(m_run - m_new);
        m_run = m_new;
        // P for the value product as an unevaluated sum of two bf16 values
        // (hi + lo carries 16 significant bits): a single bf16 P would put a
        // relative error of 2^-9 on every value it weights.
        float psum = 0.0f;
        uint32_t pk[4], pl[4];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int v = 0; v < 4; v += 2) {
                const int kk = kt * 16 + 4 * g + v;
                float p0 = none ? 0.0f : exp2f(x[kt][v] - m_new);
                float p1 = none ? 0.0f : exp2f(x[kt][v + 1] - m_new);
                psum += p0 + p1;
                const float w0 = p0 * kscale[kk], w1 = p1 * kscale[kk + 1];
                const uint32_t h = pack_bf16x2(w0, w1);
                pk[kt * 2 + v / 2] = h;
                pl[kt * 2 + v / 2] = pack_bf16x2(w0 - bf16_to_f32(h & 0xffffu), w1 - bf16_to_f32(h >> 16));
            }
        l_run = l_run * alpha + psum;
        const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
        const bf16x8 pbl = __builtin_bit_cast(bf16x8, u32x4{pl[0], pl[1], pl[2], pl[3]});
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;

        // 4. O^T += V^T P^T; lane (dim dt*16 + c16, g) needs keys 4g..4g+3 and 16+4g..16+4g+3.
        // ds_read_b64_tr_b16 within each 16-lane block hands lane i element (i & 3) of
        // the 8-byte chunk addressed by lane (i >> 2) + 4e, for e = 0..3: lane s of the
        // block addresses key 4g + (s >> 2), dims dt*16 + 4(s & 3) .. +3, so lane i
        // receives keys 4g + e at dim dt*16 + i.
        const uint8_t* vbase = lds + (4 * g + (c16 >> 2)) * T::ROWB + 8 * (c16 & 3);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const uint8_t* p0 = vbase + dt * 32;
            i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p0));
            i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(p0 + 16 * T::ROWB));
            const bf16x8 vA = __builtin_bit_cast(
                bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                              __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA, pb, o[dt], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA, pbl, o[dt], 0, 0, 0);
        }
        __syncthreads();
    }

    // finish: total row sum of this head over the 4 lane groups
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (a.nsplit == 1) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        const int64_t base = ((int64_t)r * a.H + head) * DV + 4 * g;
        if (a.out_dtype == DT_F32) {
            float* out = reinterpret_cast<float*>(a.out) + base;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(out + dt * 16) = o[dt] * inv;
        } else {
            uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + base;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                f32x4 t = o[dt] * inv;
                *reinterpret_cast<u32x2*>(out + dt * 16) = u32x2{pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3])};
            }
        }
        if (a.lse && g == 0) a.lse[(int64_t)r * a.H + head] = (m_run + log2f(l_tot)) * kLn2;
    } else {
        float* po = a.part_o + (((int64_t)r * a.nsplit + split) * a.H + head) * DV + 4 * g;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = o[dt];
        if (g == 0) {
            float* ml = a.part_ml + ((int64_t)r * a.nsplit + split) * 2 * a.H;
            ml[head] = m_run;
            ml[a.H + head] = l_tot;
        }
    }
}

// Merge the key splits of each row: m* = max m_s, w_s = 2^(m_s - m*),
// out = sum_s w_s O_s / sum_s w_s l_s, lse = (m* + log2 sum_s w_s l_s) ln 2.
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
    extern __shared__ float wts[];                  // [nsplit][H]
    const int r = blockIdx.x, tid = threadIdx.x;
    const RowKeys rk = row_keys(a, r);
    const int ns = (rk.L + a.split_keys - 1) / a.split_keys;
    const int H = a.H, DV = a.d_v;
    const float* ml = a.part_ml + (int64_t)r * a.nsplit * 2 * H;
    for (int h = tid; h < H; h += 256) {
        float M = -INFINITY;
        for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[s * 2 * H + h]);
        float Lsum = 0.0f;
        for (int s = 0; s < ns; ++s) {
            float w = ml[s * 2 * H + h] == -INFINITY ? 0.0f : exp2f(ml[s * 2 * H + h] - M);
            wts[s * H + h] = w;
            Lsum += w * ml[s * 2 * H + H + h];
        }
        const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
        for (int s = 0; s < ns; ++s) wts[s * H + h] *= inv;
        if (a.lse) a.lse[(int64_t)r * H + h] = (M + log2f(Lsum)) * kLn2;
    }
    __syncthreads();
    const float* po = a.part_o + (int64_t)r * a.nsplit * H * DV;
    for (int e = tid; e < H * DV; e += 256) {
        const int h = e / DV;
        float acc = 0.0f;
        for (int s = 0; s < ns; ++s) acc = fmaf(wts[s * H + h], po[(int64_t)s * H * DV + e], acc);
        if (a.out_dtype == DT_F32) reinterpret_cast<float*>(a.out)[(int64_t)r * H * DV + e] = acc;
        else reinterpret_cast<uint16_t*>(a.out)[(int64_t)r * H * DV + e] = (uint16_t)f32_to_bf16(acc);
    }
}

// fp32 path (tiny workloads): one workgroup per (row, head); scores in LDS.
constexpr int kF32MaxKeys = 8192;
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
    __shared__ float sc[kF32MaxKeys];
    __shared__ float red[4];
    const int h = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
    const RowKeys rk = row_keys(a, r);
    const int D = a.D;
    const float* q = reinterpret_cast<const float*>(a.q) + ((int64_t)r * a.H + h) * D;
    const float* kvd = reinterpret_cast<const float*>(a.kv_data);
    const float* wd = reinterpret_cast<const float*>(a.win_data);
    const float scale = a.scale_log2 * kLn2;
    float mx = -INFINITY;
    for (int j = tid; j < rk.L; j += 256) {
        int kind; int64_t row;
        resolve_key(a, rk, r, j, rk.L, kind, row);
        float s = -INFINITY;
        if (kind) {
            const float* kp = (kind == 1 ? kvd : wd) + row * D;
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
    for (int j = tid; j < rk.L; j += 256) {
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
        for (int j = 0; j < rk.L; ++j) {
            if (sc[j] == 0.0f) continue;
            int kind; int64_t row;
            resolve_key(a, rk, r, j, rk.L, kind, row);
            acc = fmaf(sc[j], (kind == 1 ? kvd : wd)[row * D + d], acc);
        }
        const int64_t oi = ((int64_t)r * a.H + h) * a.d_v + d;
        if (a.out_dtype == DT_F32) reinterpret_cast<float*>(a.out)[oi] = acc * inv;
        else reinterpret_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16(acc * inv);
    }
    if (a.lse && tid == 0) a.lse[(int64_t)r * a.H + h] = mx + logf(sum);
}

template <int KVD, int WD, int D, int DV, int NW>
hipError_t launch_mfma(const AttnArgs& a, hipStream_t stream) {
    dim3 grid(a.nsplit, a.num_rows);
    hipLaunchKernelGGL((attn_mfma_kernel<KVD, WD, D, DV, NW>), grid, dim3(NW * 64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(a.num_rows), dim3(256), a.nsplit * a.H * sizeof(float), stream, a);
    return hipGetLastError();
}

template <int KVD, int WD, int D, int DV>
hipError_t launch_heads(const AttnArgs& a, hipStream_t stream) {
    switch (a.H) {
    case 16: return launch_mfma<KVD, WD, D, DV, 1>(a, stream);
    case 32: return launch_mfma<KVD, WD, D, DV, 2>(a, stream);
    case 64: return launch_mfma<KVD, WD, D, DV, 4>(a, stream);
    }
    return hipErrorInvalidValue;
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

bool attn_supported(int q_dtype, int kv_dtype, int win_dtype, int H, int D, int d_v) {
    if (q_dtype == DT_F32)
        return kv_dtype == DT_F32 && (win_dtype == DT_F32 || win_dtype == DT_NONE) && D >= 1 && d_v <= D;
    if (q_dtype != DT_BF16) return false;
    if (kv_dtype != DT_BF16 && kv_dtype != DT_MXFP4) return false;
    if (win_dtype != DT_BF16 && win_dtype != DT_FP8) return false;
    if (H != 16 && H != 32 && H != 64) return false;
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
