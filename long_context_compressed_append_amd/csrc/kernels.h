// Internal interface between the host entry points (lcca_api.cpp) and the
// gfx950 kernels.  Plain structs of device pointers and sizes, validated by
// the host before a launch.
//
// Every struct carries the bounds of the indices its kernels read from
// device memory (batch, max_pos, n_blocks, total_new) and `dbg`, the device
// error word of debug builds (LCCA_DEBUG): there each such index is checked
// against its bounds before it forms an address (see checked() in device.h).
// Release builds pass dbg = nullptr and never read it.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcca {

// bits of the device error word (the public LCCA_DBG_* values)
constexpr uint32_t kDbgBlock = 1u;     // block-table entry outside the pool
constexpr uint32_t kDbgRow = 2u;       // row_seq outside the batch or row_pos outside [0, max_pos]
constexpr uint32_t kDbgChunk = 4u;     // cu_new / start_pos outside their contract

struct CompressArgs {
    const int32_t* block_table; int32_t max_blocks;
    const int32_t* cu_new; const int32_t* start_pos; int32_t batch;
    int32_t total_new; int32_t n_blocks; uint32_t* dbg;  // n_blocks: the smaller pool's
    int32_t tok_dtype;
    const void* kv_tok; const float* kv_logit; const void* ik_tok; const float* ik_logit;
    int32_t m, D, dI;
    int32_t kv_dtype; void* kv_data; void* kv_scale;
    int32_t ik_dtype; void* ik_data; void* ik_scale;     // ik_data == nullptr: no indexer stream
    int32_t win_dtype; int32_t win_cap; void* win_data; float* win_scale;   // win_data == nullptr: no window
    void* rem_kv; void* rem_ik; float* rem_kv_logit; float* rem_ik_logit;
    // per-channel-gated groups: logits [n][dim] per stream, ring logits
    // [batch][m][dim] (launch_compress_gated only)
    int32_t gated;
};

struct IndexArgs {
    const int32_t* block_table; int32_t max_blocks;
    const int32_t* row_seq; const int32_t* row_pos; int32_t num_rows;
    int32_t batch, max_pos, n_blocks; uint32_t* dbg;
    const void* q; const float* w; float s_I;
    int32_t HI, dI, m;
    int32_t key_dtype; const void* keys;
    float* logits; int64_t ld;
    // FP8 queries (q8 != 0, FP8 keys, fewer than 64 rows): each head's query
    // quantised to E4M3 with a power-of-two scale, products on the FP8 MFMA
    int32_t q8;
    // launch plan
    int32_t tiles_per_wave;      // 32-entry tiles per wave (decode) / per workgroup (prefill)
    // Decode launches ahead of the step's compress_append (fresh != 0, m <= 4):
    // row r is the one new token of its sequence (token r of the batch), and
    // an entry that token completes is not in the pool yet, so the kernel
    // forms it from the remainder ring and the token and scores it itself.
    int32_t fresh;
    const int32_t* cu_new; const int32_t* start_pos; int32_t tok_dtype;
    const void* ik_tok; const float* ik_logit; const void* rem_ik; const float* rem_ik_logit;
    // non-null: the decode kernel also adds, per row, how many of its logits
    // have each leading kTopkLeadBits-bit key digit ([rows][2^kTopkLeadBits],
    // zero before the launch; the top-k selection reads and clears it)
    uint32_t* lead_hist;
};

// leading key bits of the top-k's first (histogram) pass
constexpr int kTopkLeadBits = 12;
// top-k rows hold at most this many visible entries (bitmaps of the row in LDS)
constexpr int kTopkMaxEntries = 1 << 18;
// rows longer than kTopkSplitAbove entries are selected in two launches:
// slices of kTopkSlice entries, then their candidates
constexpr int kTopkSplitAbove = 32768;
constexpr int kTopkSlice = 16384;

struct TopkArgs {
    const int32_t* row_pos; int32_t num_rows; int32_t m;
    int32_t max_pos; uint32_t* dbg;
    const float* logits; int64_t ld; int32_t k;
    int32_t* idx;
    // two-launch selection of long rows (workspace)
    uint32_t* cand_key; int32_t* cand_idx;    // [rows][cand_stride]
    int64_t cand_stride;
    int32_t nslices, slice_len;
    // one-launch selections (kRow) of the fused decode launch: the rows'
    // leading-digit counts from the indexer, read instead of counted, then
    // cleared for the next call
    uint32_t* lead_hist;
};

// slices of a row of max_entries visible entries (1: one launch) and the
// per-row candidate stride of the workspace (elements, a multiple of 4)
int topk_slices(int max_entries);
int64_t topk_cand_stride(int max_entries, int k);

struct AttnArgs {
    const int32_t* block_table; int32_t max_blocks;
    const int32_t* row_seq; const int32_t* row_pos; int32_t num_rows;
    int32_t batch, max_pos, n_blocks; uint32_t* dbg;
    const void* q; int32_t H, D, d_v; float scale_log2;     // sm_scale * log2(e)
    int32_t m; int32_t kv_dtype; const void* kv_data; const void* kv_scale;
    const int32_t* topk; int32_t k;                         // topk == nullptr: dense over visible entries
    int32_t win_dtype; const void* win_data; const float* win_scale; int32_t win_cap, window;
    int32_t out_dtype; void* out; float* lse;
    // split plan
    int32_t nsplit, split_tiles;       // key splits per row, 32-key tiles per split
    // partial values by 16-dim tiles of d_v: [.. tile][head][16 dims]
    float* part_o;     // [rows][nsplit][d_v / 16][H][16]   (nsplit > 1, fp32 partial states)
    float* part_ml;    // [rows][nsplit][H][2]: (m, l) of each head
    // bf16 outputs: partial O / l as fp16 with a power-of-two range scale
    // per (split, head, 4 value dims); part_o is then unused
    uint16_t* part_h;  // [rows][nsplit][d_v / 16][H][16]
    float* part_sc;    // [rows][nsplit][d_v / 16][H][4]
    // FP8 queries (q8 != 0, MXFP4 pools): each head's query quantised to
    // E4M3 with a power-of-two scale; pool tiles scored by the scaled
    // FP4 x FP8 MFMA on the pool's own codes and scales
    int32_t q8;
    // P carried as a bf16 hi + lo pair (1, the default) or as bf16 alone (0)
    int32_t p_lo;
};

// Rotary embedding of dims [off, off + rd) of x [rows][heads][dim] in place
// (rope.hip): pair i is (2i, 2i+1), or (i, i + rd/2) with half_split, rotated
// by fp32(pos[r]) * freq[i] (negated with inverse).
constexpr int kRopeMaxDim = 256;
struct RopeArgs {
    void* x; int64_t rows; int32_t heads, dim, off, rd;
    const int32_t* pos;
    int32_t bf16, half_split, inverse;
    int32_t hchunk, nchunks;         // launch plan: heads per thread, head runs per row
    float freq[kRopeMaxDim / 2];
};

hipError_t launch_compress_append(const CompressArgs& a, int total_new, hipStream_t stream);
hipError_t launch_compress_gated(const CompressArgs& a, int total_new, hipStream_t stream);
hipError_t launch_index_logits(const IndexArgs& a, int max_entries, hipStream_t stream);
hipError_t launch_topk_select(TopkArgs a, int max_entries, hipStream_t stream);
// top-k selection of every row (one launch, rows of up to 32K entries, 16-byte
// aligned rows) with compress_append of the new bf16 tokens in the same launch
bool topk_compress_supported(const TopkArgs& a, int max_entries, int tok_dtype);
hipError_t launch_topk_compress(TopkArgs a, int max_entries, const CompressArgs& c, int total_new, hipStream_t stream);
hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream);
hipError_t launch_rope(RopeArgs a, hipStream_t stream);

// The device error word of debug builds on the current device (its address,
// found once per device); nullptr in release builds.
hipError_t debug_word(uint32_t** word);

// which (dtype, shape) combinations the kernels are built for
bool index_supported(int q_dtype, int key_dtype, int HI, int dI);
bool attn_supported(int q_dtype, int kv_dtype, int win_dtype, int H, int D, int d_v);

}  // namespace lcca
