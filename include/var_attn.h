/*
 * var_attn.h -- C ABI of libvarattn.so: next-scale (scale-wise) attention for
 * visual-autoregressive (VAR) generation on AMD Instinct MI355X (gfx950).
 *
 * The problem, as the source pages state it:
 *  - Next-scale prediction emits one whole h_k x w_k token grid per step, with
 *    a KV cache over the earlier scales ("ARVAR: Accelerating Visual
 *    Autoregressive Model via Attention Retrospect", Background & Motivation).
 *  - Every step attends to all tokens of all historical scales ("SparVAR:
 *    Exploring Sparsity in Visual AutoRegressive Modeling for Training-Free
 *    Acceleration", abstract).  Within the current scale every token sees every
 *    other one (the grid is predicted at once).
 *  - Classifier-free guidance runs the conditional and unconditional branches
 *    concatenated along the batch ("ARVAR ...", Key Design 1).
 *  - A block-wise sparse variant keeps attention-sink scales and a cross-scale
 *    local window found through an index mapping ("SparVAR ...", abstract).
 *  - A pruned step gathers the retained query positions, computes them, and
 *    scatters the results over an upsampled earlier output ("ARVAR ...", Key
 *    Designs 2 and 3, Equations (8)-(9)).
 *
 * Token numbering: grids are row-major and concatenated in scale order;
 * off[k] = sum_{j<k} h_j*w_j.  Scales are 0-based in this ABI.
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *    allocates nothing and never frees (var_attn_dense_split_noalloc's scratch
 *    is a static array of the library's code object); between calls it keeps
 *    only cached device properties and that array's per-device address.
 *  - Host-side argument checks run before anything is launched (some query
 *    the device's compute-unit count or a kernel's occupancy); a failed check
 *    returns its status and launches nothing.  Calls are asynchronous: they enqueue on
 *    `stream` (a hipStream_t; NULL = the legacy default stream) and return.
 *  - Errors are return codes; var_last_error() gives a thread-local detail
 *    string for the last failing call on the calling thread.
 *  - Sizes that the library cannot see (allocation extents) are the caller's
 *    contract and are stated per argument.
 */
#ifndef VAR_ATTN_H
#define VAR_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum var_status {
    VAR_OK = 0,
    VAR_ERR_NULL = 1,        /* a required pointer is NULL                          */
    VAR_ERR_SCHEDULE = 2,    /* bad scale schedule (count, sizes, token total)       */
    VAR_ERR_RANGE = 3,       /* bad scale range, batch/heads, n_sel or tile sizes    */
    VAR_ERR_UNSUPPORTED = 4, /* dtype / head_dim / tile combination not implemented  */
    VAR_ERR_STRIDE = 5,      /* stride or alignment outside what the kernels accept  */
    VAR_ERR_CAPACITY = 6,    /* col_idx capacity below n_qt * n_kt                   */
    VAR_ERR_INDEX = 7,       /* inconsistent index arguments                         */
    VAR_ERR_HIP = 8          /* the HIP runtime reported an error at launch          */
} var_status;

typedef enum var_dtype { VAR_F32 = 0, VAR_BF16 = 1 } var_dtype;

#define VAR_MAX_SCALES 32

/* Scale schedule: host arrays h[num_scales], w[num_scales] (grid rows, cols).
 * 1 <= num_scales <= VAR_MAX_SCALES, 1 <= h, w <= 4096, total tokens < 2^24.  */
typedef struct var_schedule {
    int32_t num_scales;
    const int32_t* h;
    const int32_t* w;
} var_schedule;

/* Element strides of a [batch, head, token, dim] tensor; dim stride is 1. */
typedef struct var_layout {
    int64_t batch;
    int64_t head;
    int64_t token;
} var_layout;

typedef struct var_attn_desc {
    int32_t batch;          /* B >= 1 (CFG: index 0 = cond, 1 = uncond)            */
    int32_t heads;          /* H >= 1                                              */
    int32_t head_dim;       /* D: 64 or 128 for bf16 input; 32 or 64 for f32       */
    int32_t q_scale_begin;  /* queries are tokens [off[b], off[e]) ...              */
    int32_t q_scale_end;    /* ... and keys are tokens [0, off[e])                 */
    float softmax_scale;    /* 0 => 1/sqrt(head_dim)                               */
    var_dtype in_dtype;     /* dtype of q, k, v                                    */
    var_dtype out_dtype;    /* dtype of o (bf16 in: f32 or bf16; f32 in: f32)      */
    int32_t out_at_index;   /* 0: output row i is row i of o.  1 (needs q_index):  */
                            /* output row i is written to row q_index[i] of o,     */
                            /* which then holds n_q rows; other rows of o are left */
                            /* untouched (lse stays in call order)                 */
} var_attn_desc;

typedef struct var_mask_params {
    int32_t tile_q;            /* query rows per tile (>= 1; the sparse kernel uses 64) */
    int32_t tile_k;            /* key tokens per tile (>= 1; the sparse kernel uses 64) */
    int32_t sink_scales;       /* keys in scales [0, sink_scales) are always selected   */
    int32_t local_from_scale;  /* window rule applies to key scales >= this             */
    int32_t radius_y;          /* window half-height in key-grid rows (>= 0)            */
    int32_t radius_x;          /* window half-width  in key-grid cols (>= 0)            */
} var_mask_params;

/*
 * Token extent of a call (host only, no HIP call).  For queries of scales
 * [q_scale_begin, q_scale_end): first_token = off[b], n_q = off[e] - off[b],
 * kv_len = off[e].  Any output pointer may be NULL.
 */
var_status var_schedule_extent(const var_schedule* sched, int32_t q_scale_begin, int32_t q_scale_end,
                               int64_t* first_token, int64_t* n_q, int64_t* kv_len);

/*
 * Dense block-causal next-scale attention (the definition on the SparVAR and
 * ARVAR pages above): the query at token t of scale s(t) attends to every key
 * u < off[e] with s(u) <= s(t), with O = softmax(scale * q k^T) v computed
 * exactly (online softmax, fp32 accumulation).
 *
 *  q      [B][H][n_q][D] (layout q_l): row j is token off[b] + j.
 *  k, v   [B][H][>= kv_len][D] (k_l, v_l): the KV cache; tokens [0, kv_len) read.
 *  o      [B][H][rows][D] (o_l), written; rows = n_sel if q_index else n_q.
 *  lse    NULL or [B][H][rows] contiguous fp32, written: natural-log
 *         log-sum-exp of the scaled logits (-inf for a row that sees no key).
 *  q_index NULL (then n_sel must be 0) or device int32[n_sel]: output row i is
 *         the query at position q_index[i] in [0, n_q) of q (fused gather of
 *         pruned queries, "ARVAR ...", Key Design 2).  Any order; values out of
 *         range are the caller's contract (the kernel clamps them, never
 *         reading outside q).
 * Alignment: q, k, v, o 16-byte aligned; token/head/batch strides multiples
 * of 8 elements (bf16) or 4 elements (f32).
 */
/*
 * With desc->out_at_index = 1 a pruned call writes its rows straight to their
 * places in the full output grid (the scatter of "ARVAR ...", Key Design 3,
 * Equation (9), fused into the attention epilogue); var_scatter_restore with
 * upd = NULL then fills the other rows from the upsampled base (Equation (8)),
 * and the two calls touch disjoint rows.
 */
var_status var_attn_dense(const var_schedule* sched, const var_attn_desc* desc,
                          const void* q, var_layout q_l, const void* k, var_layout k_l,
                          const void* v, var_layout v_l, void* o, var_layout o_l,
                          float* lse, const int32_t* q_index, int32_t n_sel, void* stream);

/*
 * Key-split variants of var_attn_dense and var_attn_block_sparse, for launches
 * whose (batch, head, query tile) work items leave compute units idle in
 * their last round: the middle steps of a generation (the "SparVAR ..." and
 * "ARVAR ..." pages above: each step attends to every earlier scale, so a
 * step's key range grows while its query grid is still small).  The result
 * is the same attention; only the order of the floating-point sums differs.
 * The work items that fill whole rounds of the device's resident workgroups
 * (compute units times workgroups per unit) run unsplit; each remaining item
 * (every item, when there are fewer than one round's worth) is split into
 * n_splits parts, each taking an equal share of its key tiles (dense) or of
 * each 64-row mask row's kept tiles (sparse); every part writes its rows'
 * normalised O and LSE in fp32 to the workspace, and a second launch combines
 * them:
 *   O = sum_s exp(LSE_s - M) O_s / sum_s exp(LSE_s - M),  LSE = M + log(sum ...),
 *   M = max_s LSE_s  (a part in which a row sees no key has LSE_s = -inf).
 *  n_splits  1..8; 1 is exactly var_attn_dense / var_attn_block_sparse (the
 *            workspace is then not used and may be NULL).  > 1 needs bf16 input.
 *  workspace device memory, 16-byte aligned, owned by the caller, of
 *            n_splits*P*(D+1)*4 bytes, P the rows of the split work items:
 *            the (batch, head, row) rows, in that order, from the first row
 *            of the first split item on (P depends on the device's compute
 *            units; var_attn_split_plan reports the bytes, and
 *            n_splits*B*H*rows*(D+1)*4 is always enough).  Its contents on
 *            entry do not matter and on return are unspecified.  Calls that
 *            share a workspace must be ordered on one stream.
 *  Other arguments as in var_attn_dense / var_attn_block_sparse.
 * Errors: VAR_ERR_RANGE for n_splits outside 1..8, VAR_ERR_UNSUPPORTED for a
 * split of f32 input, VAR_ERR_NULL / VAR_ERR_STRIDE / VAR_ERR_CAPACITY for a
 * missing, misaligned or short workspace.
 */
var_status var_attn_dense_split(const var_schedule* sched, const var_attn_desc* desc,
                                const void* q, var_layout q_l, const void* k, var_layout k_l,
                                const void* v, var_layout v_l, void* o, var_layout o_l,
                                float* lse, const int32_t* q_index, int32_t n_sel,
                                int32_t n_splits, void* workspace, int64_t workspace_bytes, void* stream);
var_status var_attn_block_sparse_split(const var_schedule* sched, const var_attn_desc* desc,
                                       const void* q, var_layout q_l, const void* k, var_layout k_l,
                                       const void* v, var_layout v_l, void* o, var_layout o_l,
                                       float* lse, const int32_t* q_index, int32_t n_sel,
                                       const int32_t* row_ptr, const int32_t* col_idx,
                                       int32_t tile_q, int32_t tile_k, int32_t n_splits,
                                       void* workspace, int64_t workspace_bytes, void* stream);

/*
 * var_attn_dense_split without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the fp32 partials go to a static device array of
 * the library, VAR_NOALLOC_SCRATCH_BYTES per device (held from library load to
 * process end; its address is looked up once per device).  The call itself
 * allocates nothing.  A call whose split partials (the bytes
 * var_attn_split_plan reports for it) exceed the array returns
 * VAR_ERR_CAPACITY before anything is launched (it only queries the
 * device's compute-unit count and occupancy); n_splits = 1 uses no scratch.  Every
 * call on a device shares that device's array: calls that overlap on one
 * device (other streams, other threads) race and must be ordered by the
 * caller.  Other arguments and errors as in var_attn_dense_split.
 */
#define VAR_NOALLOC_SCRATCH_BYTES (64ll << 20)
var_status var_attn_dense_split_noalloc(const var_schedule* sched, const var_attn_desc* desc,
                                        const void* q, var_layout q_l, const void* k, var_layout k_l,
                                        const void* v, var_layout v_l, void* o, var_layout o_l,
                                        float* lse, const int32_t* q_index, int32_t n_sel,
                                        int32_t n_splits, void* stream);

/*
 * Split count for a call (host only; reads the current device's compute-unit
 * count, 256 if it cannot): the fewest splits whose modelled time is within
 * 3% of the lowest (the unsplit rounds, then rounds of parts over the
 * resident workgroups times key tiles per part, plus the combining launch and
 * its workspace traffic).  A dense work item is 128 query rows at head_dim
 * 128 when all of the call's 128-row items fit one round of the compute
 * units, else 256 rows.  kv_tiles_hint: 64-key tiles a work item visits
 * (0 = ceil(kv_len / 64), the dense count; pass the mean kept tiles per mask
 * row for a sparse call; the model still counts the dense kernel's work
 * items, one workgroup per compute unit, so for sparse calls it is a rougher
 * guide).  Writes *n_splits and the workspace bytes a dense or block-sparse
 * call with that count needs on this device (either pointer may be NULL).
 * n_sel as in var_attn_dense (0 = no gather).  f32 input always gives 1 and
 * 0 bytes.
 */
var_status var_attn_split_plan(const var_schedule* sched, const var_attn_desc* desc, int32_t n_sel,
                               int32_t kv_tiles_hint, int32_t* n_splits, int64_t* workspace_bytes);

/*
 * Tile mask of the block-sparse variant ("SparVAR ...", abstract: attention
 * sinks, cross-scale locality through an index map, block-wise sparsity).
 * A (query, key) pair is selected when s(key) <= s(query) and either
 * s(key) < sink_scales, or s(key) >= local_from_scale and, with j = s(key),
 * q = s(query):  |y_q*h_j - y_k*h_q| <= radius_y*h_q  and
 *                |x_q*w_j - x_k*w_q| <= radius_x*w_q  (exact integers).
 * Tile (r, c) is kept when some selected pair has its query among rows
 * [r*tile_q, (r+1)*tile_q) of the call (rows as in var_attn_dense, i.e. after
 * the q_index gather) and its key in tokens [c*tile_k, (c+1)*tile_k) of
 * [0, kv_len).  Output CSR, one list shared by every (batch, head):
 *  row_ptr  device int32[n_qt + 1]; col_idx device int32[col_capacity] with
 *  col_capacity >= n_qt * n_kt (the buffer doubles as the build's staging
 *  area; entries past row_ptr[n_qt] are left unspecified).  Each row lists
 *  its kept key tiles in ascending order.
 *  n_qt = ceil(rows / tile_q), n_kt = ceil(kv_len / tile_k).
 * q_index as in var_attn_dense (device, positions in [0, n_q)).
 */
var_status var_tile_mask_dims(const var_schedule* sched, int32_t q_scale_begin, int32_t q_scale_end,
                              const var_mask_params* mp, int32_t n_sel_or_0,
                              int32_t* n_qt, int32_t* n_kt);
var_status var_build_tile_mask(const var_schedule* sched, int32_t q_scale_begin, int32_t q_scale_end,
                               const var_mask_params* mp, const int32_t* q_index, int32_t n_sel,
                               int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                               void* stream);

/*
 * Several tile masks of one schedule and one rule at once: a generation's
 * masks depend on positions (and the retained index lists) only, so they are
 * all known up front.  calls[i] asks for what var_build_tile_mask builds for
 * its own query range, gather and CSR arrays, under the same contract per
 * call; the result equals n_calls calls of var_build_tile_mask.  The rows of
 * every call are built by one launch and the lists compacted by a second (a
 * workgroup per call), so the calls run side by side instead of one after
 * another.  1 <= n_calls <= VAR_MAX_MASK_CALLS; every call is checked on the
 * host before anything is launched (a failed check names the call).  The
 * CSR arrays of different calls must not overlap.
 */
#define VAR_MAX_MASK_CALLS 16
typedef struct var_tile_mask_call {
    int32_t q_scale_begin;
    int32_t q_scale_end;
    const int32_t* q_index;   /* device, positions in [0, n_q), or NULL */
    int32_t n_sel;            /* entries of q_index (0 without) */
    int32_t* row_ptr;         /* device int32[n_qt + 1] */
    int32_t* col_idx;         /* device int32[col_capacity] */
    int64_t col_capacity;     /* >= n_qt * n_kt */
} var_tile_mask_call;
var_status var_build_tile_masks(const var_schedule* sched, const var_mask_params* mp,
                                const var_tile_mask_call* calls, int32_t n_calls, void* stream);

/*
 * Block-sparse next-scale attention: var_attn_dense restricted to the kept
 * tiles of a CSR tile mask (as produced by var_build_tile_mask).  Inside a
 * kept tile every block-causally visible pair is attended.  tile_q = tile_k
 * = 64 only.  Arguments as in var_attn_dense; row_ptr / col_idx are device
 * arrays with n_qt + 1 and row_ptr[n_qt] entries.  A row whose kept tiles
 * hold no visible key gets O = 0 and LSE = -inf.
 * CSR contract (the caller's; the arrays are on the device and not checked
 * on the host): row_ptr[0] = 0, row_ptr non-decreasing, row_ptr[n_qt] at most
 * the capacity of col_idx; each row's columns strictly ascending, in
 * [0, n_kt).  Within that contract each listed tile is attended once.  With
 * row_ptr inside the contract, any column values keep every access in
 * bounds: a column outside [0, n_kt) is clamped into it, a column repeated
 * right after itself counts once, and any other repeat (out of order) counts
 * its tile again.
 */
var_status var_attn_block_sparse(const var_schedule* sched, const var_attn_desc* desc,
                                 const void* q, var_layout q_l, const void* k, var_layout k_l,
                                 const void* v, var_layout v_l, void* o, var_layout o_l,
                                 float* lse, const int32_t* q_index, int32_t n_sel,
                                 const int32_t* row_ptr, const int32_t* col_idx,
                                 int32_t tile_q, int32_t tile_k, void* stream);

/*
 * A pruned block-sparse step and its structural reconstruction in one
 * launch ("ARVAR ...", Key Design 3, Equations (8)-(9)): the attention of
 * var_attn_block_sparse with desc->out_at_index = 1 writes output row i to
 * row q_index[i] of the step's full grid o, and workgroups of the same
 * launch fill every other row of o from the nearest-upsampled base (source
 * (floor(y*h_in/h), floor(x*w_in/w)), the rule of var_scatter_restore), in
 * the compute-unit slots the attention leaves free (when it leaves fewer
 * than 64 free, the fill runs as a second launch right after the attention
 * on the same stream).  The result equals
 * var_attn_block_sparse (out_at_index = 1) followed by var_scatter_restore
 * with upd = NULL, bit for bit.
 *  desc    bf16 input, out_at_index = 1, one step: q_scale_end =
 *          q_scale_begin + 1, whose grid h x w (from sched) is the output grid.
 *  o       [B][H][h*w][D] (o_l) of out_dtype, every row written.
 *  base    [B][H][>= h_in*w_in][D] (base_l) of out_dtype, read only.
 *  q_index device int32[n_sel], strictly ascending, in [0, h*w) (NULL allowed
 *          when n_sel = 0: then every row comes from the base).
 *  err_flag NULL or a device int32 the caller has zeroed: 1 is ORed in for an
 *          index out of range, 2 for a pair not strictly ascending; rows are
 *          then unspecified but every access stays in bounds.
 * Other arguments as in var_attn_block_sparse (its CSR contract included;
 * no key splits).  o and base 16-byte aligned, all their strides multiples
 * of 16 bytes, token strides >= D, and (for batch > 1) batch stride = heads
 * x head stride, else VAR_ERR_STRIDE.  Nothing is launched on an error.
 */
var_status var_attn_block_sparse_restore(const var_schedule* sched, const var_attn_desc* desc,
                                         const void* q, var_layout q_l, const void* k, var_layout k_l,
                                         const void* v, var_layout v_l, void* o, var_layout o_l,
                                         float* lse, const int32_t* q_index, int32_t n_sel,
                                         const int32_t* row_ptr, const int32_t* col_idx,
                                         int32_t tile_q, int32_t tile_k, const void* base, var_layout base_l,
                                         int32_t h_in, int32_t w_in, int32_t* err_flag, void* stream);

/*
 * Saliency of the positions of one (small) step, the signal of attention-guided
 * pruning ("ARVAR ...", Key Design 2: the attention of an earlier step of the
 * same layer is reduced to one score per position of its grid; A Worked
 * Example: the source step lies M = 3 steps before the pruned one).  The page
 * leaves the reduction axis, the normalisation and the head aggregation
 * open; this call takes the self-attention block of the step's attention
 * weights P (rows normalised over every key the query sees) and returns, per
 * (batch, head), the mean over the step's queries of each own-scale column:
 *   saliency[b][h][u] = (1/n_s) * sum_i exp(scale * q_i . k_{off[s]+u} - lse[b][h][i])
 * for u < n_s = h_s*w_s.
 *  desc   batch, heads, head_dim (64 or 128), softmax_scale as for
 *         var_attn_dense; q_scale_end must be q_scale_begin + 1 (= s); bf16
 *         input only (out_dtype is ignored).
 *  q, k   as in var_attn_dense for that call (q row j = token off[s] + j).
 *  lse    device fp32 [B][H][n_s], contiguous: the natural-log LSE that
 *         var_attn_dense returned for the same call (not re-derived here).
 *  saliency device fp32 [B][H][n_s], contiguous, written.
 * Errors: VAR_ERR_RANGE for a range of more than one scale; VAR_ERR_UNSUPPORTED
 * for f32 input or other head dims.
 */
var_status var_attn_saliency(const var_schedule* sched, const var_attn_desc* desc,
                             const void* q, var_layout q_l, const void* k, var_layout k_l,
                             const float* lse, float* saliency, void* stream);

/*
 * Top-K choice of the retained positions of a pruned step ("ARVAR ...", Key
 * Design 2: the saliency map is interpolated to the current grid and Top-K
 * gives the indices to gather; Key Design 3 scatters them back).
 * score(t) for t = (y, x) of the h_dst x w_dst grid is
 *   S[floor(y*h_src/h_dst) * w_src + floor(x*w_src/w_dst)],
 *   S[u] = saliency[0][u] + saliency[1][u] + ... (fp32, in map order)
 * (nearest interpolation, the rule of var_scatter_restore).  The n_keep
 * positions with the largest score are written to q_index in ascending
 * order; among equal scores lower positions win.  -0.0 counts as 0; scores
 * must not be NaN (with NaN the result is still n_keep distinct ascending
 * positions, in an unspecified choice).
 *  saliency device fp32 [maps][h_src*w_src] contiguous (e.g. the output of
 *           var_attn_saliency with maps = B*H); h_src*w_src <= 8192.
 *  q_index  device int32[n_keep], written; n_keep in [0, h_dst*w_dst]
 *           (0 launches nothing).  Usable directly as the q_index of the
 *           attention, mask and scatter calls.
 * One workgroup; meant for grids of a few thousand positions.
 */
var_status var_select_topk(int32_t maps, const float* saliency, int32_t h_src, int32_t w_src,
                           int32_t h_dst, int32_t w_dst, int32_t n_keep, int32_t* q_index, void* stream);

/*
 * Sparse pattern of a later step predicted from a decision scale ("SparVAR
 * ...", abstract: the sparse attention pattern of later high-resolution
 * scales is predicted dynamically from a sparse decision scale, and made
 * self-similar to it through an index mapping between scales).  The abstract
 * fixes no formulas; the three calls below take this reading, with 64x64
 * tiles throughout:
 *
 * var_attn_block_mass: attention mass of the decision step d (one scale,
 * bf16, head_dim 64 or 128; q, k, desc as for var_attn_dense of that step):
 *   mass[b][h][r][c] = sum_{i in rows 64r..64r+63} sum_{u in tokens 64c..64c+63, u < off[d+1]}
 *                      exp(scale * q_i . k_u - lse[b][h][i])
 * with lse the LSE var_attn_dense returned for the same call (device fp32
 * [B][H][n_d] contiguous).  mass: device fp32 [B][H][ceil(n_d/64)][ceil(off[d+1]/64)],
 * contiguous, written.  n_d <= 8192.
 */
var_status var_attn_block_mass(const var_schedule* sched, const var_attn_desc* desc,
                               const void* q, var_layout q_l, const void* k, var_layout k_l,
                               const float* lse, float* mass, void* stream);

/*
 * var_decision_tiles: per row (map, r) of mass [maps][n_qt][n_kt] (device fp32),
 * the key tiles in order of decreasing mass (equal masses: lower c first) are
 * kept while the mass already kept is below tau * total, the sums in fp32, in
 * that order, the total in ascending c.  kept: device uint8 [maps][n_qt][n_kt]
 * (1 = kept), written.  0 <= tau <= 1; n_kt <= 1024; masses must not be NaN.
 */
var_status var_decision_tiles(int32_t maps, int32_t n_qt, int32_t n_kt, const float* mass, float tau,
                              uint8_t* kept, void* stream);

/*
 * var_mapped_tile_mask: per-map tile mask of step T (queries = scale T, keys
 * [0, off[T+1])) from kept_d [maps][ceil(n_d/64)][ceil(off[d+1]/64)] of the
 * decision step d <= T.  A query (y, x) of scale T stands for position
 * (floor(y*h_d/h_T), floor(x*w_d/w_T)) of scale d; a key of a scale j <= d for
 * itself; a key (y, x) of a scale j > d for (floor(y*h_d/h_j), floor(x*w_d/w_j))
 * of scale d.  Tile (R, C) is kept when some query of R and key of C stand
 * for a kept decision pair.  Output: one CSR per map, row_ptr device int32
 * [maps][n_qt + 1] and col_idx device int32 [maps][col_stride] (col_stride >=
 * n_qt * n_kt: the buffer doubles as staging), n_qt = ceil(n_T/64),
 * n_kt = ceil(off[T+1]/64), lists ascending.  Limits: ceil(n_d/64) and
 * ceil(off[d+1]/64) <= 1024, n_kt <= 8192.
 */
var_status var_mapped_tile_mask(const var_schedule* sched, int32_t decision_scale, int32_t step,
                                int32_t maps, const uint8_t* kept_d, int32_t* row_ptr, int32_t* col_idx,
                                int64_t col_stride, void* stream);

/*
 * var_attn_block_sparse with one CSR per (batch, head) (e.g. from
 * var_mapped_tile_mask with maps = B*H): map m = b*H + h reads row_ptr
 * + m*(n_qt + 1) and col_idx + m*col_stride.  bf16 input, 64x64 tiles.
 * Other arguments as in var_attn_block_sparse.
 */
var_status var_attn_block_sparse_heads(const var_schedule* sched, const var_attn_desc* desc,
                                       const void* q, var_layout q_l, const void* k, var_layout k_l,
                                       const void* v, var_layout v_l, void* o, var_layout o_l,
                                       float* lse, const int32_t* q_index, int32_t n_sel,
                                       const int32_t* row_ptr, const int32_t* col_idx,
                                       int64_t col_stride, void* stream);

/*
 * Low-bit (FP8) attention ("LiteVAR: Compressing Visual Autoregressive
 * Modelling with Efficient Attention and Quantization", abstract: the data
 * precision of a VAR model is redundant and low-bit quantisation keeps its
 * quality).  The record names no format, operand or granularity; these calls
 * compute the logits from queries and keys in OCP e4m3 (1 sign, 4 exponent
 * bits with bias 7, 3 mantissa bits, subnormals, largest finite 448, no
 * infinities; 0x7F and 0xFF are NaN) with one fp32 scale per 64-token tile,
 * value = e4m3 value * scale.  The attention weights and v stay bf16.
 *
 * var_quantize_e4m3: x is bf16 [batch][heads][tokens][head_dim] (layout x_l,
 * finite values).  Tile j of map m = b*heads + h holds tokens
 * [64j, min(64j + 64, tokens)); for every tile with 64(j+1) > first_token:
 *   amax = max |x| over the tile (1 if all zero), inv = 448 / amax (fp32,
 *   correctly rounded), code = e4m3(x * inv) (fp32 product, round to nearest
 *   even, magnitudes above 448 -> 448), scale[m*scale_stride + j] = amax / 448.
 * Tiles before first_token / 64 are left untouched (codes and scales), so a
 * growing key cache requantises only the tiles its new tokens reach.
 *  codes  device uint8, same shape, layout c_l (strides in bytes, multiples
 *         of 16), written.
 *  scale  device fp32 [batch*heads][scale_stride], scale_stride >=
 *         ceil(tokens/64), written.
 *  0 <= first_token <= tokens (= tokens: nothing to do; pointers may then be
 *  NULL); head_dim a multiple of 16 in [16, 256]; batch*heads <= 65535.
 *
 * var_attn_dense_e4m3: var_attn_dense_split with the logits taken from e4m3
 * queries and keys.  k is e4m3 codes with tile scales (e.g. from
 * var_quantize_e4m3 of the key cache); q is bf16 and is quantised inside the
 * call, rows [64j, 64j + 64) of the call (after the q_index gather) forming
 * one group with the rule of var_quantize_e4m3.  With qs the scale of the
 * group of output row i and m = b*heads + h, the logit of row i and key u is
 *   softmax_scale * qs * k_scale[m*k_scale_stride + u/64] * (q_codes . k_codes),
 * i.e. attention of the dequantised queries and keys.  The e4m3 matrix
 * instruction does not round its sums like fp32: its error reached 2^-11.8
 * of the sum of the product magnitudes for codes spread over the whole e4m3
 * range (the worst case measured on gfx950; 2^-14.6 for normally distributed
 * codes), so a logit can move by up to 2^-11.8 * softmax_scale * qs * ks *
 * sum_d |q_d k_d|: around 2e-3 at softmax_scale = 1/sqrt(128) on unit data
 * in the worst case, about 3e-4 typically.
 *  desc   in_dtype must be VAR_BF16 (the dtype of q and v); head_dim 128;
 *         out_dtype f32 or bf16.
 *  k      device uint8 codes [B][H][>= kv_len][128], layout k_l (strides in
 *         bytes, multiples of 16).
 *  k_scale device fp32 [B*H][k_scale_stride], k_scale_stride >= ceil(kv_len/64),
 *         positive.
 *  Other arguments as in var_attn_dense_split.
 * var_attn_block_sparse_e4m3: the block-sparse call (64x64 tiles) with the
 * same e4m3 logits; col_stride 0 takes one CSR shared by every (batch, head)
 * (as var_attn_block_sparse), col_stride > 0 one CSR per (batch, head) as in
 * var_attn_block_sparse_heads.
 * Errors: VAR_ERR_UNSUPPORTED for another head_dim or in_dtype, VAR_ERR_NULL
 * for a missing k_scale, VAR_ERR_STRIDE for code strides that are not
 * multiples of 16 bytes or a scale stride below the key tiles; otherwise as
 * the bf16 calls.
 */
var_status var_quantize_e4m3(int32_t batch, int32_t heads, int32_t tokens, int32_t head_dim,
                             const void* x, var_layout x_l, uint8_t* codes, var_layout c_l,
                             float* scale, int64_t scale_stride, int32_t first_token, void* stream);
var_status var_attn_dense_e4m3(const var_schedule* sched, const var_attn_desc* desc,
                               const void* q, var_layout q_l, const uint8_t* k, var_layout k_l,
                               const float* k_scale, int64_t k_scale_stride,
                               const void* v, var_layout v_l, void* o, var_layout o_l,
                               float* lse, const int32_t* q_index, int32_t n_sel,
                               int32_t n_splits, void* workspace, int64_t workspace_bytes, void* stream);
var_status var_attn_block_sparse_e4m3(const var_schedule* sched, const var_attn_desc* desc,
                                      const void* q, var_layout q_l, const uint8_t* k, var_layout k_l,
                                      const float* k_scale, int64_t k_scale_stride,
                                      const void* v, var_layout v_l, void* o, var_layout o_l,
                                      float* lse, const int32_t* q_index, int32_t n_sel,
                                      const int32_t* row_ptr, const int32_t* col_idx,
                                      int64_t col_stride, void* stream);

/*
 * Structural reconstruction of a pruned grid ("ARVAR ...", Key Design 3,
 * Equations (8)-(9)): out = Scatter(Up(base; h_out, w_out), q_index, upd).
 * Up is nearest neighbour with source (floor(y*h_in/h_out), floor(x*w_in/w_out));
 * Scatter overwrites row q_index[i] with upd row i.  Rows are copied bit for
 * bit.  For each map m in [0, maps) (e.g. m = b*H + h):
 *   base  rows at base + m*base_map_stride + t*base_row_stride, t < h_in*w_in
 *   upd   rows at upd  + m*upd_map_stride  + i*upd_row_stride,  i < n_sel
 *   out   rows at out  + m*out_map_stride  + t*out_row_stride,  t < h_out*w_out
 * each row holding row_elems contiguous elements of `dtype`; strides are in
 * elements.  q_index: device int32[n_sel], strictly ascending, in
 * [0, h_out*w_out).  err_flag: NULL or a device int32 the caller has zeroed;
 * the kernel ORs in 1 for an out-of-range index and 2 for a non-ascending
 * (duplicate or unsorted) pair; rows are then unspecified but every access
 * stays in bounds.
 * upd = NULL with n_sel > 0: the rows q_index[i] of out are left untouched
 * (written by an attention call with out_at_index = 1) and only the other
 * rows are filled from the upsampled base; the two calls may then run in
 * either order or concurrently.
 */
var_status var_scatter_restore(int32_t maps, int32_t row_elems, var_dtype dtype,
                               const void* base, int64_t base_map_stride, int64_t base_row_stride,
                               int32_t h_in, int32_t w_in,
                               const void* upd, int64_t upd_map_stride, int64_t upd_row_stride,
                               const int32_t* q_index, int32_t n_sel,
                               void* out, int64_t out_map_stride, int64_t out_row_stride,
                               int32_t h_out, int32_t w_out, int32_t* err_flag, void* stream);

/*
 * Compute units and peak engine clock (kHz) of the calling thread's current
 * device, as the key-split plan sees them (read once per device from the
 * device properties).  Either pointer may be NULL.  VAR_ERR_HIP when there is
 * no device.
 */
var_status var_device_info(int32_t* compute_units, int32_t* max_clock_khz);

/* Static name of a status code. */
const char* var_status_string(var_status s);
/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* var_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VAR_ATTN_H */
