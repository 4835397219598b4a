// Internal interface between the C-ABI host layer (var_attn_api.cpp) and the
// gfx950 kernels.  Not installed; the public interface is include/var_attn.h.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

#include "../../include/var_attn.h"

namespace varattn {

struct ScatterParams {
    const unsigned char* base;
    const unsigned char* upd;
    unsigned char* out;
    const int32_t* q_index;
    int32_t* err_flag;
    int64_t base_map_stride, base_row_stride;   // bytes
    int64_t upd_map_stride, upd_row_stride;     // bytes
    int64_t out_map_stride, out_row_stride;     // bytes
    int32_t maps, row_bytes, n_sel;
    int32_t h_in, w_in, h_out, w_out;
    int32_t unit;     // copy width in bytes (16, 4 or 2) dividing rows, strides and pointers
};

// Everything one attention launch needs.  Passed by value as kernel argument.
struct AttnParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const int32_t* q_index;   // nullable
    const int32_t* row_ptr;   // sparse only
    const int32_t* col_idx;   // sparse only
    int64_t q_sb, q_sh, q_st;
    int64_t k_sb, k_sh, k_st;
    int64_t v_sb, v_sh, v_st;
    int64_t o_sb, o_sh, o_st;
    int32_t B, H;
    int32_t n_rows;      // output rows per (b, h): n_sel or n_q
    int32_t n_q;         // query tokens of the call
    int32_t q_first;     // token index of query row 0
    int32_t kv_len;      // keys [0, kv_len)
    int32_t n_qtiles;    // query tiles per (b, h) of this launch
    int32_t num_scales;
    int32_t step_mode;   // every query lies in the last scale => key limit is kv_len
    int32_t out_at_index;   // output row i goes to row q_index[i] of o
    float scale;         // softmax scale
    float scale_log2;    // scale * log2(e)
    int32_t scale_end[VAR_MAX_SCALES];  // off[s + 1]
    // key splits (bf16 kernel): work items (batch, head, query tile), numbered
    // bh * n_qtiles + tile, below split_from run whole; with n_splits > 1 each
    // later item runs as n_splits workgroups, each taking an equal share of
    // its key tiles and writing fp32 O and LSE to part_o [n_splits][part_rows][D]
    // / part_lse [n_splits][part_rows]; a merge launch then writes their o and
    // lse.  The split items' rows are those of the flattened (b*H + h)*n_rows +
    // row numbering from part_first on (item split_from's first row), so
    // part_rows = B*H*n_rows - part_first.  n_splits == 1: split_from = items.
    int32_t n_splits;
    int32_t split_from;
    float* part_o;
    float* part_lse;
    int64_t part_first;
    int64_t part_rows;
    // per-(batch, head) CSR (block-sparse): element strides between the maps'
    // row_ptr / col_idx arrays (0: one CSR shared by every (batch, head))
    int64_t rp_bh_stride, ci_bh_stride;
    // e4m3 keys (launch_attn_fp8 only): dequantisation scale of key tile
    // key / 64 at k_scale[bh * k_scale_stride + key / 64]
    const float* k_scale;
    int64_t k_scale_stride;
    // reconstruction in the same launch (block-sparse bf16, out_at_index): the
    // last rs_wgs workgroups of the grid fill the rows of o that q_index does
    // not name from the nearest-upsampled base (rs.upd NULL), in groups of
    // rs_rows_per_group rows; 0 for every other launch
    ScatterParams rs;
    int32_t rs_wgs;
    int32_t rs_rows_per_group;
};

// Row of o that output row `row` of an attention call is written to: itself,
// or (out_at_index) its gathered position, clamped like the gather.
__device__ __forceinline__ int out_row_of(const AttnParams& p, int row) {
    if (!p.out_at_index) return row;
    const int pos = p.q_index[row];
    return pos < 0 ? 0 : (pos >= p.n_q ? p.n_q - 1 : pos);
}

// Largest key-split count of a launch.
constexpr int kMaxSplits = 8;

struct MaskParams {
    const int32_t* q_index;   // nullable
    int32_t* row_ptr;
    int32_t* col_idx;
    int32_t n_rows, n_q, q_first, kv_len;
    int32_t n_qt, n_kt;
    int32_t tile_q, tile_k;
    int32_t sink_scales, local_from_scale, radius_y, radius_x;
    int32_t num_scales;
    int32_t off[VAR_MAX_SCALES + 1];
    int32_t h[VAR_MAX_SCALES];
    int32_t w[VAR_MAX_SCALES];
    int64_t rp_map_stride, ci_map_stride;   // per-map CSR strides of the compaction (0: one map)
};


// Launchers: return the hipError_t of the launch.
// rows_per_tile: attn_bf16_rows_per_tile of the call (it selects the kernel);
// cus: the device's compute units (a block-sparse launch that fits one round
// of them runs one workgroup per unit with a deeper ring).
// restore: a block-sparse unsplit launch with p.rs set, followed by
// reconstruction workgroups (the launcher sets rs_wgs and rs_rows_per_group).
hipError_t launch_attn_bf16(const AttnParams& p, int head_dim, bool out_bf16, bool sparse, int rows_per_tile,
                            int cus, hipStream_t s, bool restore = false);
// The same attention with k as e4m3 codes (k_scale set) and q quantised to
// e4m3 in the kernel, one scale per 64-row tile of the call; v bf16.
hipError_t launch_attn_fp8(const AttnParams& p, int head_dim, bool out_bf16, bool sparse, hipStream_t s);
hipError_t launch_attn_f32(const AttnParams& p, int head_dim, bool sparse, hipStream_t s);
// e4m3 quantisation with one scale per (batch, head, 64-token tile).
struct QuantParams {
    const void* x;            // bf16 [B][H][tokens][D] (element strides)
    uint8_t* codes;           // e4m3 codes, same shape (element = byte strides)
    float* scale;             // [B*H][scale_stride] dequantisation scales of the tiles
    int64_t scale_stride;
    int64_t x_sb, x_sh, x_st;
    int64_t c_sb, c_sh, c_st;
    int32_t H, maps, tokens, D;
    int32_t tile_first;       // first tile written (tiles tile_first .. ceil(tokens / 64) - 1)
};
hipError_t launch_quant_e4m3(const QuantParams& p, hipStream_t s);

// Saliency of one step's own-scale keys (column means of its attention weights).
struct SaliencyParams {
    const void* q;        // bf16 queries of the step, row j = token key_first + j
    const void* k;        // bf16 key cache
    const float* lse;     // [B*H][n_s] natural-log LSE of the step's attention rows
    float* sal;           // [B*H][n_s] output
    int64_t q_sb, q_sh, q_st;
    int64_t k_sb, k_sh, k_st;
    int32_t B, H;
    int32_t n_s;          // tokens of the step's scale (queries = own-scale keys)
    int32_t key_first;    // token index of the scale's first key
    int32_t n_kb;         // 64-key blocks per (b, h)
    float scale_log2;     // softmax scale * log2(e)
};

// Largest source grid of the Top-K selection (source scores live in LDS).
constexpr int kSelectMaxSrc = 8192;
// Destination grids up to this size keep their keys in LDS during the selection.
constexpr int kSelectDstCache = 6912;

struct SelectParams {
    const float* sal;     // [maps][h_src*w_src]
    int32_t* q_index;     // [n_keep] output, ascending
    int32_t maps, h_src, w_src, h_dst, w_dst, n_keep;
};

// Decision-scale sparse pattern (per-head tile masks predicted by index mapping).
constexpr int kMassMaxRows = 8192;           // rows of the decision step
constexpr int kDecisionMaxTiles = 1024;      // key tiles of the decision step
constexpr int kDecisionMaxRowTiles = 1024;   // row tiles of the decision step
constexpr int kMappedMaxTiles = 8192;        // key tiles of the predicted step

struct MassParams {
    const void* q;        // bf16 queries of the decision step (row j = token off[d] + j)
    const void* k;        // bf16 key cache
    const float* lse;     // [B*H][n_rows] LSE of the decision step's attention
    float* mass;          // [B*H][ceil(n_rows/64)][n_kt] output
    int64_t q_sb, q_sh, q_st;
    int64_t k_sb, k_sh, k_st;
    int32_t B, H, n_rows, kv_len, n_kt;
    float scale_log2;
};

struct DecisionParams {
    const float* mass;    // [rows][n_kt]
    unsigned char* kept;  // [rows][n_kt] output (0 / 1)
    int32_t n_kt;
    float tau;
};

struct MappedParams {
    const unsigned char* kept_d;   // [maps][n_qt_d][n_kt_d]
    int32_t* row_ptr;              // [maps] x rp_map_stride
    int32_t* col_idx;              // [maps] x ci_map_stride
    int64_t rp_map_stride, ci_map_stride;
    int32_t d, T;
    int32_t n_qt, n_kt;            // tiles of step T
    int32_t n_qt_d, n_kt_d;        // tiles of the decision step
    int32_t off[VAR_MAX_SCALES + 1];
    int32_t h[VAR_MAX_SCALES];
    int32_t w[VAR_MAX_SCALES];
};

hipError_t launch_tile_mask(const MaskParams& p, hipStream_t s);
hipError_t launch_block_mass(const MassParams& p, int head_dim, hipStream_t s);
hipError_t launch_decision(const DecisionParams& p, int rows, hipStream_t s);
hipError_t launch_mapped_mask(const MappedParams& p, int maps, hipStream_t s);
// Several tile masks of one schedule and one rule (var_build_tile_masks):
// the schedule and rule once, then per call its query range, gather and
// CSR; built by one rows launch over every call's query tiles and one
// compaction launch with a workgroup per call.
constexpr int kMaxMaskBatch = 16;
struct MaskCall {
    const int32_t* q_index;   // nullable
    int32_t* row_ptr;
    int32_t* col_idx;
    int32_t n_rows, n_q, q_first, kv_len;
    int32_t n_qt, n_kt;
    int32_t num_scales;       // q_scale_end of the call
};
struct MaskBatch {
    MaskCall c[kMaxMaskBatch];
    int32_t first_block[kMaxMaskBatch + 1];   // rows-launch workgroups of call i: [first_block[i], first_block[i + 1])
    int32_t n_calls;
    int32_t tile_q, tile_k;
    int32_t sink_scales, local_from_scale, radius_y, radius_x;
    int32_t off[VAR_MAX_SCALES + 1];
    int32_t h[VAR_MAX_SCALES];
    int32_t w[VAR_MAX_SCALES];
};
hipError_t launch_tile_mask_batch(const MaskBatch& b, hipStream_t s);

// The compaction of launch_tile_mask alone, one workgroup per map.
hipError_t launch_mask_compact(const MaskParams& p, int maps, hipStream_t s);
hipError_t launch_saliency(const SaliencyParams& p, int head_dim, hipStream_t s);
hipError_t launch_select_topk(const SelectParams& p, hipStream_t s);
hipError_t launch_scatter(const ScatterParams& p, hipStream_t s);
hipError_t launch_zero_i32(int32_t* p, hipStream_t s);

// Query-tile height (rows per workgroup) of a bf16 launch over bh maps of
// `rows` rows each on a device of `cus` compute units: 128 for block-sparse
// attention; for dense attention 128 at head_dim 128 when those work items fit
// one round of the device's resident workgroups, else 256.
int attn_bf16_rows_per_tile(int head_dim, bool sparse, int64_t bh, int64_t rows, int cus);
// The same for the e4m3 kernels: 128 block-sparse, 256 dense.
int attn_fp8_rows_per_tile(bool sparse);
// Workgroups of the bf16 / e4m3 attention kernel that one compute unit holds
// at once (from the runtime's occupancy query; 1 when it cannot say).
int attn_bf16_resident_wgs(int head_dim, bool out_bf16, bool sparse, int rows_per_tile);
int attn_fp8_resident_wgs(bool out_bf16, bool sparse);
constexpr int kF32RowsPerTile = 64;

}  // namespace varattn
