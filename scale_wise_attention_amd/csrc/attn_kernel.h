// Block-causal next-scale attention for gfx950: bf16 (or e4m3 q / k, QK8)
// in, fp32 accumulate.
//
// For every query row of the call: O = softmax(scale * q K^T) V over the keys
// the row may see, i.e. all keys of its own and earlier scales ("SparVAR:
// Exploring Sparsity in Visual AutoRegressive Modeling for Training-Free
// Acceleration", abstract: each step attends to all tokens of the historical
// scales; "ARVAR: Accelerating Visual Autoregressive Model via Attention
// Retrospect", Background & Motivation: a whole grid per step with a KV
// cache).  Key u is visible to token t iff u < end of t's scale: one key
// limit per query.  The block-sparse variant visits only the kept key tiles
// of each 64-row query tile ("SparVAR ...", abstract: block-wise sparse
// attention); q_index fuses the gather of pruned queries ("ARVAR ...", Key
// Design 2).
//
// Design (dense: one workgroup = 256 query rows of one (batch, head), 4 waves
// of 64 rows, one wave per SIMD, or, at head_dim 128 for launches whose work
// items fit one round of the device, 128 rows as 4 waves of 32; block-sparse:
// 128 rows, two workgroups per compute unit, as 4 waves of 32 rows (two waves
// per SIMD) at head_dim 128 and 2 waves of 64 rows at 64):
//  * Each wave owns QB 32-query column blocks (QB = 2: 64 queries; QB = 1:
//    32).  S^T = K Q^T is computed with v_mfma_f32_32x32x16_bf16 (keys on M,
//    queries on N), so a lane holds 16 logits of each of its queries and lane
//    l^32 holds the other 16 of every 32-key block.  With two blocks every K
//    operand read from LDS feeds two MFMAs, halving LDS traffic per FLOP; one
//    block shortens a wave's tile (half the MFMAs) and leaves it at most 256
//    registers, so in a block-sparse workgroup two waves share a SIMD and
//    one's LDS reads and softmax run under the other's MFMAs.
//  * The same registers, rounded to bf16, are the B operand of
//    O^T += V^T P^T (d on M, queries on N, keys on K).  The MFMA's k order is
//    matched by permuting keys inside the V^T tile in LDS, so P never moves
//    between lanes.  Q stays in AGPRs for the whole key loop; the O
//    accumulators are VGPRs (VGPR-form MFMAs) and the K / V^T operands read
//    from LDS are handed to the MFMAs from AGPRs.
//  * Tiles that need no mask run a branch-free body, unrolled at compile
//    time into one slot per MFMA: the QK chains block by block, then the PV
//    MFMAs, with the weights of each key pair computed in three stages
//    (scale+shift, exp2, pack) spread over the slots in between.  K goes
//    straight from global memory into LDS (global_load_lds); V goes through
//    registers and is written transposed under the last PV chunk.  A dense
//    walk keeps a 4-slot LDS ring two tiles ahead and runs these tiles in
//    pairs, one barrier per pair; a block-sparse walk keeps 2 slots, one
//    tile ahead, one barrier per tile.  The first tile and masked tiles run
//    a general body.
//  * Softmax in the log2 domain (scale*log2(e) folded into one FMA before
//    v_exp_f32) against a fixed reference max per row: the max of the first
//    tile in which the row sees a key.  Later weights may exceed 1 (fp32 and
//    bf16 keep the full exponent range), so the accumulators are never
//    rescaled, the loop body has no control flow around them and, once
//    every row has its reference, no row max is computed at all.  A row
//    whose sum ends up above 2^100 (or non-finite) had logits far above its
//    reference: then the workgroup recomputes, first the exact row maxima
//    (QK only), then the weights against them (all <= 1).  Row sums
//    accumulate the bf16-rounded weights with v_dot2 (the same weights that
//    multiply V).
//  * Block-sparse: a workgroup covers 2 consecutive 64-row query tiles; it
//    walks the merged (union) list of their kept key tiles, and the waves of
//    each query tile compute only the tiles of that tile's own list (on the
//    others they just stage their share of the next V tile).
//  * Key splits (n_splits > 1): the work items that fill whole rounds of the
//    device's resident workgroups run unsplit; each remaining item runs as
//    n_splits workgroups, each with an equal share of its key tiles, which
//    write fp32 partial O and LSE; split_merge_kernel combines them with
//    log-sum-exp weights.
//  * Workgroup ids are remapped so the query tiles of one (batch, head) run
//    on one XCD and share its L2 for K and V.
//  * QK8 (e4m3 logits, the low-bit data precision of "LiteVAR: Compressing
//    Visual Autoregressive Modelling with Efficient Attention and
//    Quantization"): K arrives as e4m3 codes with one scale per 64-key tile;
//    each wave quantises its 64 bf16 query rows (one group, one scale) on
//    load; S^T comes from v_mfma_f32_32x32x64_f8f6f4 (2 MFMAs per 32x32
//    block), and the tile's log2-domain factor is the product of the two
//    scales.  Weights, V and the rest are as above.
#pragma once

#include <hip/hip_runtime.h>

#include <climits>
#include <type_traits>
#include <utility>

#include "e4m3.h"
#include "kernels.h"
#include "scatter_rows.h"

namespace varattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int KT = 64;                 // keys per tile (= sparse tile width)
// query rows per workgroup when a wave owns QB 32-row query blocks:
// block-sparse 128 (two 64-row mask rows; the workgroup walks the union of
// the two rows' kept tiles, and two workgroups share a compute unit); dense
// 256 with QB = 2 (4 waves of 64 rows, the throughput shape) and 128 with
// QB = 1 (4 waves of 32 rows, one per SIMD: for launches whose work items fit
// one round of the device, where the latency of a tile counts, not the rate)
template <bool SPARSE, int QB>
constexpr int rows_per_wg() { return SPARSE ? 2 * KT : (QB == 1 ? 2 * KT : 4 * KT); }
// waves per workgroup
template <bool SPARSE, int QB>
constexpr int waves_per_wg() { return rows_per_wg<SPARSE, QB>() / (32 * QB); }
constexpr float kSumLimit = 0x1p100f;  // a row sum above this triggers the exact recompute

// Work of workgroup wg (of nwg): work item `item`, key split `split`, and
// whether the item runs whole.  Items below split_from run whole; every later
// item runs as `splits` pieces (pieces of one item are consecutive).  The
// dispatcher places workgroup i on XCD i % 8 and starts an XCD's workgroups in
// order, so each XCD takes an equal share of the whole items first and then an
// equal share of the pieces, each share a contiguous range: neighbouring items
// belong to one (batch, head) and share its K and V in that XCD's L2.
__device__ __forceinline__ void decode_work(int wg, int nwg, int split_from, int splits, int& item, int& split,
                                            bool& whole) {
    // (branch-free, results in scalar registers: the values are uniform)
    const int x = wg & 7, j = wg >> 3;
    const int fq = split_from >> 3, fr = split_from & 7;
    const int n_whole = fq + (x < fr ? 1 : 0);   // whole items on this XCD
    const int q = nwg >> 3, r = nwg & 7;
    const bool w = j < n_whole;
    const int piece = max(x * (q - fq) + min(x, r) - min(x, fr) + (j - n_whole), 0);
    const int pdiv = piece / splits;
    item = __builtin_amdgcn_readfirstlane(w ? x * fq + min(x, fr) + j : split_from + pdiv);
    split = __builtin_amdgcn_readfirstlane(w ? 0 : piece - pdiv * splits);
    whole = w;
}

__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m));
    return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = max(v, __shfl_xor(v, m));
    return v;
}
__device__ __forceinline__ float swap_halves(float v) { return __shfl_xor(v, 32); }

// K tile with ROWB-byte rows: row r (key), 16-byte chunk c -> stored at
// chunk c ^ k_swz(r), so that the 16 rows one operand read touches land in
// 16 different 16-byte bank groups
template <int ROWB>
__device__ __forceinline__ int k_swz(int r) {
    static_assert(ROWB == 64 || ROWB == 128 || ROWB == 256, "K row of 64, 128 or 256 bytes");
    if constexpr (ROWB == 256) return r & 15;
    else if constexpr (ROWB == 128) return (r >> 1) & 7;
    else return (r >> 2) & 3;
}
// V^T tile: row d holds 64 keys (128 bytes, 16-byte chunks c = 0..7); rows
// 2m and 2m+1 share a 256-byte line of 16 slots.  Chunk c of row d goes to slot
// ((d ^ c) & 1) * 8 + (c ^ H(m)) with H(m) = (m + ((m >> 3) & 1)) & 7, so that
//  - an operand read (16 lanes: 16 consecutive d, one chunk) and
//  - a staging write (32 lanes: 8 d of one parity x 2 chunks x two 8-byte halves)
// each touch every LDS bank once, and the swizzle depends on d & 31 only (the
// 32-row block of d is a constant offset).
__device__ __forceinline__ int v_addr(int d, int c) {
    const int m = d >> 1;
    const int h = (m + ((m >> 3) & 1)) & 7;
    return m * 256 + ((((d ^ c) & 1) << 3) | ((c ^ h) & 7)) * 16;
}

// low halves of a and b -> (a.lo, b.lo); high halves -> (a.hi, b.hi): one v_perm_b32 each
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
// round-to-nearest-even pair conversion: one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// A global-memory pointer every lane holds, moved to SGPRs: loads then take
// the scalar base + 32-bit lane offset form instead of 64-bit vector adds.
typedef __attribute__((address_space(1))) const char gchar;
__device__ __forceinline__ const gchar* uniform_ptr(const gchar* q) {
    const uint64_t v = reinterpret_cast<uint64_t>(q);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const gchar*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float max3(float a, float b, float c) { return __builtin_fmaxf(a, __builtin_fmaxf(b, c)); }

template <int V>
struct IntC {
    static constexpr int value = V;
};

template <bool B>
struct BoolC {
    static constexpr bool value = B;
};

// calls f(std::integral_constant<int, I>) for I = 0..N-1 (every index a constant)
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Slots of the branch-free tile body (one MFMA each): the QK MFMAs of the 2*QB
// 32x32 S^T blocks (half h, query block qb) run chain by chain (SK k-steps:
// slots (QB*h+qb)*SK .. +SK-1), then the PV MFMAs (chunk C, d block mb, query
// block qb; NP = QB * (d blocks) per chunk) at slot 2*QB*SK + C*NP + QB*mb + qb.
// Weight pair i (half i / (8 QB), block (i / 8) % QB, chunk (i >> 2) & 1, pair
// i & 3) takes three stages in slots at[i], at[i]+1, at[i]+2: from two slots
// after its S^T block is complete, and done before the first PV MFMA that
// reads it.  Pairs are spread evenly over
// the slots in between (earliest deadline first), at most CAP first stages
// per slot.
template <int SK, int NP, int CAP, int QB>
struct WeightSlots {
    static constexpr int NPAIR = 16 * QB;      // weight pairs of a lane per tile
    static constexpr int NS = 2 * QB * SK + 4 * NP;
    int at[NPAIR];
    static constexpr int half_of(int i) { return i / (8 * QB); }
    static constexpr int qb_of(int i) { return (i / 8) % QB; }
    static constexpr int release(int i) { return (QB * half_of(i) + qb_of(i) + 1) * SK + 1; }
    static constexpr int deadline(int i) {   // the stage-3 slot must come before this one
        return 2 * QB * SK + (2 * half_of(i) + ((i >> 2) & 1)) * NP + qb_of(i);
    }
    constexpr WeightSlots() : at{} {
        const int cap = CAP;
        int first = NS, last = 0;
        bool done[NPAIR] = {};
        for (int i = 0; i < NPAIR; ++i) {
            first = release(i) < first ? release(i) : first;
            last = deadline(i) - 3 > last ? deadline(i) - 3 : last;
        }
        const int span = last - first + 1;
        int placed = 0;
        for (int m = 0; m < NS; ++m) {
            int k = 0;
            bool tried[NPAIR] = {};
            while (k < cap) {
                int best = -1;
                for (int i = 0; i < NPAIR; ++i)
                    if (!done[i] && !tried[i] && release(i) <= m && (best < 0 || deadline(i) < deadline(best))) best = i;
                if (best < 0) break;
                tried[best] = true;
                const bool urgent = deadline(best) - 3 - m <= 0;
                const int quota = ((m - first + 1) * NPAIR + span - 1) / span;
                if (urgent || placed < quota) {
                    at[best] = m;
                    done[best] = true;
                    ++placed;
                    ++k;
                }
            }
        }
    }
    constexpr bool valid() const {
        for (int i = 0; i < NPAIR; ++i)
            if (at[i] < release(i) || at[i] + 2 >= deadline(i)) return false;
        return true;
    }
};

// One entry of the key-tile walk: tile index (-1 = end), the waves that use
// it and (e4m3 keys) the tile's dequantisation scale, loaded when the entry
// is made, a few tiles before it is used.
struct TileEnt {
    int tile;
    int mask;
    float ks;
};

// QK8: k is e4m3 codes with one scale per 64-key tile, each wave quantises
// its 64 bf16 query rows to e4m3 (one scale), and S^T comes from
// v_mfma_f32_32x32x64_f8f6f4 (64 deep per k-step); V stays bf16.
// WIDE: the 4-slot ring (two tiles ahead) and tile pairs, one workgroup per
// compute unit: every dense walk, and block-sparse launches whose workgroups
// all fit one round of the device (the others keep two workgroups per unit
// with a 2-slot ring)
// RESTORE: the last p.rs_wgs workgroups of the grid do not attend; they fill
// the rows of the full output grid that the (out_at_index) pruned call does
// not write, from the nearest-upsampled base, in the slots the attention's
// workgroups leave free
template <int D, bool OUT_BF16, bool SPARSE, bool QK8, int QB, bool WIDE = !SPARSE, bool RESTORE = false>
__global__ __launch_bounds__((waves_per_wg<SPARSE, QB>() * 64), ((SPARSE && QB == 1 && !WIDE) ? 2 : 1)) void attn_kernel(const AttnParams p) {
    static_assert(QB == 1 || QB == 2, "one or two 32-row query blocks per wave");
    static_assert(!RESTORE || (SPARSE && !QK8), "reconstruction rides on bf16 block-sparse launches");
    static_assert(WIDE || SPARSE, "dense walks use the 4-slot ring");
    static_assert(!QK8 || QB == 2, "e4m3 queries are quantised per 64 rows: one wave's rows");
    constexpr int NW = waves_per_wg<SPARSE, QB>();   // waves per workgroup
    constexpr int NT = NW * 64;                      // threads per workgroup
    constexpr int QW = 32 * QB;                      // query rows per wave
    constexpr int QT = rows_per_wg<SPARSE, QB>();    // query rows per workgroup
    constexpr int NL = QT / KT;                      // block-sparse: kept-tile lists (64-row mask rows) per workgroup
    constexpr int EK = QK8 ? 1 : 2;            // bytes per k element (q is always bf16)
    constexpr int ROWB = D * EK;               // bytes per K row
    constexpr int KCH = ROWB / 16;             // 16-byte chunks per K row
    constexpr int K_BYTES = KT * ROWB;
    constexpr int V_BYTES = KT * D * 2;
    constexpr int V_UNITS = (KT / 4) * (D / 4);
    constexpr int V_PER_T = V_UNITS / NT;      // 4x4 V blocks per thread
    static_assert(K_BYTES % (1024 * NW) == 0, "K tile split into 1 KB wave segments");
    static_assert(V_PER_T * NT == V_UNITS, "V tile split");
    constexpr int SK = QK8 ? D / 64 : D / 16;  // k-steps of S^T = K Q^T
    static_assert(!QK8 || D == 128, "e4m3 q / k with head_dim 128 only (one k-step of 64 leaves no slots for the weights)");
    // a Q / K MFMA operand: 32 e4m3 codes or 8 bf16 values per lane
    typedef typename std::conditional<QK8, i32x8, bf16x8>::type qop;
    constexpr int MO = D / 32;                 // 32-row blocks of O^T

    // LDS ring of K and V^T tiles: 4 slots (two tiles ahead, pairs of tiles
    // per barrier) in a wide walk, 2 (one tile ahead) in a block-sparse walk
    // that shares its compute unit
    constexpr int RING = WIDE ? 4 : 2;
    constexpr int AHEAD = RING / 2;
    __shared__ __attribute__((aligned(16))) unsigned char smem[RING * K_BYTES + RING * V_BYTES];
    unsigned char* const Kbuf = smem;
    unsigned char* const Vbuf = smem + RING * K_BYTES;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;      // lane half
    const int n = lane & 31;      // column inside a 32-query block

    // workgroups of the attention itself (those after them reconstruct)
    const int n_attn = RESTORE ? (int)gridDim.x - p.rs_wgs : (int)gridDim.x;
    if constexpr (RESTORE) {
        static_assert(kScatterPasses * NT * (int)sizeof(int) <= (int)sizeof(smem), "row-group marks fit the ring");
        if ((int)blockIdx.x >= n_attn) {
            const int wg = (int)blockIdx.x - n_attn;
            scatter_check_index<NT>(p.rs, wg, p.rs_wgs);
            scatter_groups<16, NT>(p.rs, p.rs_rows_per_group, wg, p.rs_wgs, reinterpret_cast<int*>(smem));
            return;
        }
    }

    // work item = (batch, head, query tile), whole or one of its key splits
    int item, split;
    bool whole;
    decode_work(blockIdx.x, n_attn, p.split_from, p.n_splits, item, split, whole);
    // this workgroup's share count (1: the whole item).  The later tests use
    // this integer, not the flag: a flag kept for them cost the key loop
    // about a dozen registers (moved through AGPRs every tile).
    const int n_sp = __builtin_amdgcn_readfirstlane(whole ? 1 : p.n_splits);
    const int qtile = item % p.n_qtiles;
    const int bh = item / p.n_qtiles;
    const int b = bh / p.H;
    const int h = bh - b * p.H;

    // ---- this lane's query rows (one per 32-row block) -----------------
    int my_row[QB], klim[QB];
    bool row_valid[QB];
    float c2q[QB];   // log2-domain logit scale of each of the lane's queries
    qop qreg[QB][SK];
    uint32_t qraw[QB][QK8 ? SK : 1][4][4];   // e4m3 path: the lane's bf16 query values
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        my_row[qb] = qtile * QT + wave * QW + 32 * qb + n;
        row_valid[qb] = my_row[qb] < p.n_rows;
        const int row_c = row_valid[qb] ? my_row[qb] : (p.n_rows - 1);
        int pos = p.q_index ? p.q_index[row_c] : row_c;
        pos = pos < 0 ? 0 : (pos >= p.n_q ? p.n_q - 1 : pos);
        const int tok = p.q_first + pos;
        int kl = p.kv_len;
        if (!p.step_mode) {
#pragma unroll
            for (int s = VAR_MAX_SCALES - 1; s >= 0; --s)
                if (s < p.num_scales && tok < p.scale_end[s]) kl = p.scale_end[s];
        }
        klim[qb] = kl;
        c2q[qb] = p.scale_log2;
        const unsigned char* qp = reinterpret_cast<const unsigned char*>(p.q) +
                                  (b * p.q_sb + h * p.q_sh + (int64_t)pos * p.q_st) * 2;
#pragma unroll
        for (int ks = 0; ks < SK; ++ks) {
            // lane half g holds k = 8g..8g+7 of the bf16 step (16 deep) or
            // 32g..32g+31 of the e4m3 step (64 deep)
            if constexpr (QK8) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u32x4 t = *reinterpret_cast<const u32x4*>(qp + 2 * (64 * ks + 32 * g + 8 * c));
                    qraw[qb][ks][c][0] = t.x, qraw[qb][ks][c][1] = t.y, qraw[qb][ks][c][2] = t.z, qraw[qb][ks][c][3] = t.w;
                }
            } else {
                qreg[qb][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 32 * ks + 16 * g));
            }
        }
    }
    const unsigned char* kp = reinterpret_cast<const unsigned char*>(p.k) + (b * p.k_sb + h * p.k_sh) * EK;
    const __bf16* vp = reinterpret_cast<const __bf16*>(p.v) + b * p.v_sb + h * p.v_sh;
    const int kv_last = p.kv_len - 1;

    u32x2 vreg[V_PER_T][4];

    // Per-lane byte offsets inside a tile (rows of a 64-key tile; the host
    // guarantees 64 rows of K and V fit 32-bit offsets).  Every offset is
    // formed as a non-negative 32-bit value before it is added to a tile's
    // 64-bit base.  Interior tiles use precomputed offsets; the tail tile
    // clamps rows to kv_len-1 (those keys are masked later).
    constexpr int ROWS_PER_SEG = 1024 / ROWB;
    constexpr int SEG_PER_WAVE = K_BYTES / 1024 / NW;
    const gchar* const kbytes = uniform_ptr((const gchar*)(reinterpret_cast<uintptr_t>(kp)));
    const gchar* const vbytes = uniform_ptr((const gchar*)(reinterpret_cast<uintptr_t>(vp)));
    const uint32_t k_st_bytes = (uint32_t)p.k_st * EK;
    const uint32_t v_st_bytes = (uint32_t)p.v_st * 2u;
    uint32_t k_col[SEG_PER_WAVE];   // byte offset of this lane's 16-byte chunk in its row
    int k_row[SEG_PER_WAVE];        // row of the tile this lane fetches
#pragma unroll
    for (int i = 0; i < SEG_PER_WAVE; ++i) {
        const int seg = wave * SEG_PER_WAVE + i;
        k_row[i] = seg * ROWS_PER_SEG + lane / KCH;
        k_col[i] = (uint32_t)(((lane % KCH) ^ k_swz<ROWB>(k_row[i])) * 16);
    }
    uint32_t k_full[SEG_PER_WAVE];  // offsets of an interior (full) tile
#pragma unroll
    for (int i = 0; i < SEG_PER_WAVE; ++i) k_full[i] = (uint32_t)k_row[i] * k_st_bytes + k_col[i];
    // V staging unit u: keys 4kg..4kg+3 x columns 4dg..4dg+3 (one 8-byte load per
    // key).  Within the 16-key block kb the 4-key groups g4 = 0..3 are stored in
    // the order {0, 2, 1, 3} (the order in which a lane's weights come out of
    // S^T): group g4 goes to chunk 2kb + (g4 & 1), 8-byte half g4 >> 1.  The bits
    // of u are (from the lowest): half, dg mod 8, chunk parity, then dg / 8 and kb.
    auto v_unit = [&](int u, int& dg, int& kg, int& chunk, int& half) __attribute__((always_inline)) {
        const int c0 = (u >> 4) & 1, r = u >> 5;
        const int kb = r / (D / 32);
        half = u & 1;
        dg = 8 * (r % (D / 32)) + ((u >> 1) & 7);
        kg = 4 * kb + 2 * half + c0;
        chunk = 2 * kb + c0;
    };
    uint32_t v_col[V_PER_T];
    int v_row[V_PER_T];
#pragma unroll
    for (int j = 0; j < V_PER_T; ++j) {
        int dg, kg, chunk, half;
        v_unit(tid + NT * j, dg, kg, chunk, half);
        v_row[j] = 4 * kg;
        v_col[j] = (uint32_t)(8 * dg);
    }
    uint32_t v_full[V_PER_T];       // lane offsets of an interior (full) tile
#pragma unroll
    for (int j = 0; j < V_PER_T; ++j) v_full[j] = (uint32_t)v_row[j] * v_st_bytes + v_col[j];
    // a loop-invariant lane offset made opaque at its use, so that the
    // address is formed there as scalar base + 32-bit offset (one instruction)
    auto lane_off = [](uint32_t o) __attribute__((always_inline)) -> uint32_t {
        asm volatile("" : "+v"(o));
        return o;
    };
    // K tile straight from global memory into LDS (no registers): each lane of a
    // wave writes 16 bytes at lane*16 of the wave's 1 KB segment, so the
    // swizzle is applied by choosing which global chunk each lane fetches.
    auto load_k = [&](int kbase, int slot) __attribute__((always_inline)) {
        unsigned char* Ks = Kbuf + slot * K_BYTES;
        const gchar* tb = uniform_ptr(kbytes + (int64_t)kbase * p.k_st * EK);
        auto issue = [&](int i, uint32_t off) __attribute__((always_inline)) {
            __builtin_amdgcn_global_load_lds(tb + off, (__attribute__((address_space(3))) void*)(Ks + (wave * SEG_PER_WAVE + i) * 1024),
                                             16, 0, 0);
        };
        if (kbase + KT <= p.kv_len) {
#pragma unroll
            for (int i = 0; i < SEG_PER_WAVE; ++i) issue(i, lane_off(k_full[i]));
        } else {
            const int last = kv_last - kbase;   // last valid row of this tile (< KT here)
#pragma unroll
            for (int i = 0; i < SEG_PER_WAVE; ++i) issue(i, (uint32_t)min(k_row[i], last) * k_st_bytes + k_col[i]);
        }
    };
    auto load_v = [&](int kbase) __attribute__((always_inline)) {
        const gchar* tb = uniform_ptr(vbytes + (int64_t)kbase * p.v_st * 2);
        if (kbase + KT <= p.kv_len) {
#pragma unroll
            for (int j = 0; j < V_PER_T; ++j) {
                const uint32_t o = lane_off(v_full[j]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    vreg[j][r] = *reinterpret_cast<const __attribute__((address_space(1))) u32x2*>(
                        uniform_ptr(tb + (uint32_t)r * v_st_bytes) + o);
            }
        } else {
            const int last = kv_last - kbase;
#pragma unroll
            for (int j = 0; j < V_PER_T; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t off = (uint32_t)min(v_row[j] + r, last) * v_st_bytes + v_col[j];
                    vreg[j][r] = *reinterpret_cast<const __attribute__((address_space(1))) u32x2*>(tb + off);
                }
        }
    };
    // one 4-key x 1-column piece (row i of the 4x4 block j) of the V^T staging
    auto store_v_piece = [&](int slot, int j, int i) __attribute__((always_inline)) {
        unsigned char* Vs = Vbuf + slot * V_BYTES;
        int dg, kg, chunk, half;
        v_unit(tid + NT * j, dg, kg, chunk, half);
        const u32x2* a = vreg[j];
        u32x2 outv;
        if (i == 0) outv = u32x2{pack_lo(a[0].x, a[1].x), pack_lo(a[2].x, a[3].x)};
        if (i == 1) outv = u32x2{pack_hi(a[0].x, a[1].x), pack_hi(a[2].x, a[3].x)};
        if (i == 2) outv = u32x2{pack_lo(a[0].y, a[1].y), pack_lo(a[2].y, a[3].y)};
        if (i == 3) outv = u32x2{pack_hi(a[0].y, a[1].y), pack_hi(a[2].y, a[3].y)};
        *reinterpret_cast<u32x2*>(Vs + v_addr(4 * dg + i, chunk) + half * 8) = outv;
    };
    auto store_v = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < V_PER_T; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) store_v_piece(slot, j, i);
    };

    // The first key tile of an unsplit dense walk is tile 0 (keys [0, 64),
    // always present): its K DMA and V loads are issued now, so that their
    // latency overlaps the Q loads' (a small step is little more than these
    // two round trips).  The walk's prologue then skips them.
    bool first_tile_preloaded = false;
    if constexpr (!SPARSE) {
        if (n_sp == 1) {
            load_k(0, 0);
            load_v(0);
            first_tile_preloaded = true;
        }
    }
    if constexpr (QK8) {
        // The wave's 64 rows are one 64-row tile of the call: quantise it to
        // e4m3 with one scale (amax / 448; rows past n_rows repeat the last
        // row and leave the maximum unchanged), in the operand layout.
        uint32_t mx = 0u;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int ks = 0; ks < SK; ++ks)
#pragma unroll
                for (int c = 0; c < 4; ++c) mx = max(mx, bf16x8_absmax_bits(qraw[qb][ks][c]));
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, m));
        const float amax = mx ? __uint_as_float(mx) : 1.0f;
        const float inv = __fdiv_rn(448.0f, amax);
        const float sq = __fdiv_rn(amax, 448.0f);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            c2q[qb] = p.scale_log2 * sq;
#pragma unroll
            for (int ks = 0; ks < SK; ++ks) {
                uint32_t cw[8];
#pragma unroll
                for (int c = 0; c < 4; ++c) bf16x8_to_e4m3(qraw[qb][ks][c], inv, cw[2 * c], cw[2 * c + 1]);
                qreg[qb][ks] = i32x8{(int)cw[0], (int)cw[1], (int)cw[2], (int)cw[3],
                                     (int)cw[4], (int)cw[5], (int)cw[6], (int)cw[7]};
                asm volatile("" : "+a"(qreg[qb][ks]));
            }
        }
    } else {
        // Q is only ever an MFMA operand: keep it in AGPRs (MFMAs read them
        // directly), which leaves the VGPRs to the softmax and the loads
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int ks = 0; ks < SK; ++ks) asm volatile("" : "+a"(qreg[qb][ks]));
    }
    int kl_min = klim[0], kl_max = klim[0];
#pragma unroll
    for (int qb = 1; qb < QB; ++qb) {
        kl_min = min(kl_min, klim[qb]);
        kl_max = max(kl_max, klim[qb]);
    }
    const int w_kmin = __builtin_amdgcn_readfirstlane(wave_min_i(kl_min));
    const int w_kmax = __builtin_amdgcn_readfirstlane(wave_max_i(kl_max));

    // ---- key-tile walk (workgroup-uniform) ------------------------------
    const int n_kt_all = (p.kv_len + KT - 1) / KT;
    int dense_begin = 0, dense_end = 0;   // dense: tiles [dense_begin, dense_end)
    int dense_next = 0;
    int lbeg[NL], lptr[NL], lend[NL], lhead[NL];   // sparse: one list per 64-row mask row
    const int my_list = wave * QW / KT;             // the list of this wave's rows
    // this (batch, head)'s CSR, read through the constant address space: the
    // launch never writes it and every read is workgroup-uniform, so the
    // reads go through the scalar path into scalar registers
    typedef const __attribute__((address_space(4))) int32_t* csr_ptr;
    const csr_ptr rowp = (csr_ptr)(p.row_ptr + bh * p.rp_bh_stride);
    const csr_ptr coli = (csr_ptr)(p.col_idx + bh * p.ci_bh_stride);
    if constexpr (SPARSE) {
        const int n_qt = (p.n_rows + KT - 1) / KT;
#pragma unroll
        for (int w = 0; w < NL; ++w) {
            const int r = qtile * NL + w;
            const int b0 = r < n_qt ? rowp[r] : 0;
            const int cnt = r < n_qt ? rowp[r + 1] - b0 : 0;
            // key split: an equal share of this row's kept tiles (in order; the
            // host bounds cnt * n_splits below 2^31)
            lbeg[w] = n_sp > 1 ? b0 + cnt * split / n_sp : b0;
            lend[w] = n_sp > 1 ? b0 + cnt * (split + 1) / n_sp : b0 + cnt;
            // a share that starts inside a run of one repeated column leaves
            // the run to the share that holds its first entry
            while (lbeg[w] > b0 && lbeg[w] < lend[w] && coli[lbeg[w]] == coli[lbeg[w] - 1]) ++lbeg[w];
            lptr[w] = lbeg[w];
            lhead[w] = lptr[w] < lend[w] ? coli[lptr[w]] : INT_MAX;
        }
    }
    // workgroup reductions in LDS words of their own (a K DMA may be in flight)
    __shared__ int wg_words[3 * NW];
    // wide block-sparse walks: each wave's "rows without a reference" flag,
    // posted per tile (two sets, by tile parity) until no wave has one
    __shared__ int ref_words[2][NW];
    int wg_kmin;   // smallest key limit in the workgroup: tiles below it need no mask
    {
        int* red = wg_words;
        if (lane == 0) {
            red[wave] = w_kmax;
            red[NW + wave] = w_kmin;
        }
        __syncthreads();
        int m = red[0], mn = red[NW];
#pragma unroll
        for (int i = 1; i < NW; ++i) {
            m = max(m, red[i]);
            mn = min(mn, red[NW + i]);
        }
        __syncthreads();
        if constexpr (!SPARSE) {
            const int n_t = (m + KT - 1) / KT;   // key split: an equal share of the tiles
            dense_begin = n_sp > 1 ? __builtin_amdgcn_readfirstlane(n_t * split / n_sp) : 0;
            dense_end = n_sp > 1 ? __builtin_amdgcn_readfirstlane(n_t * (split + 1) / n_sp) : n_t;
            dense_next = dense_begin;
        }
        wg_kmin = __builtin_amdgcn_readfirstlane(mn);
    }
    auto next_tile = [&]() __attribute__((always_inline)) -> TileEnt {
        TileEnt e;
        if constexpr (SPARSE) {
            int c = INT_MAX;
#pragma unroll
            for (int w = 0; w < NL; ++w) c = min(c, lhead[w]);
            e.tile = -1;
            e.mask = 0;
            if (c != INT_MAX) {
#pragma unroll
                for (int w = 0; w < NL; ++w) {
                    if (lhead[w] == c) {
                        e.mask |= 1 << w;
                        // (a column repeated right after itself is taken once)
                        do {
                            ++lptr[w];
                            lhead[w] = lptr[w] < lend[w] ? coli[lptr[w]] : INT_MAX;
                        } while (lhead[w] == c);
                    }
                }
                // a column outside [0, n_kt) cannot come from the mask builder; clamp so loads stay in bounds
                e.tile = min(max(c, 0), n_kt_all - 1);
            }
        } else {
            e.tile = dense_next < dense_end ? dense_next : -1;
            e.mask = (1 << NL) - 1;
            ++dense_next;
        }
        e.ks = 1.f;
        if constexpr (QK8) {
            // (uniform and never written by the launch: a scalar load, as for the CSR)
            typedef const __attribute__((address_space(4))) float* scale_ptr;
            if (e.tile >= 0) e.ks = ((scale_ptr)p.k_scale)[bh * p.k_scale_stride + e.tile];
        }
        return e;
    };
    auto reset_walk = [&]() __attribute__((always_inline)) {
        if constexpr (SPARSE) {
#pragma unroll
            for (int w = 0; w < NL; ++w) {
                lptr[w] = lbeg[w];
                lhead[w] = lptr[w] < lend[w] ? coli[lptr[w]] : INT_MAX;
            }
        } else {
            dense_next = dense_begin;
        }
    };
    auto mine = [&](const TileEnt& e) __attribute__((always_inline)) -> bool {
        if constexpr (SPARSE) return e.tile >= 0 && ((e.mask >> my_list) & 1);
        else return e.tile >= 0 && e.tile * KT < w_kmax;
    };

    // S^T of one 32-key half: s[qb] holds keys kb0 + 8(r/4) + 4g + (r%4) of query 32qb + n.
    // The K operand of k-step ks for key row r of a tile in LDS (same lane
    // layout as the Q operand)
    auto k_operand = [&](const unsigned char* Ks, int r, int ks) __attribute__((always_inline)) -> qop {
        if constexpr (QK8) {
            const u32x4 lo = *reinterpret_cast<const u32x4*>(Ks + (r * KCH + ((4 * ks + 2 * g) ^ k_swz<ROWB>(r))) * 16);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(Ks + (r * KCH + ((4 * ks + 2 * g + 1) ^ k_swz<ROWB>(r))) * 16);
            return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
            return *reinterpret_cast<const bf16x8*>(Ks + (r * KCH + ((2 * ks + g) ^ k_swz<ROWB>(r))) * 16);
        }
    };
    // one k-step of S^T += K Q^T (e4m3 x e4m3 or bf16 x bf16, fp32 accumulate)
    auto qk_step = [](const qop& a, const qop& q, const f32x16& c) __attribute__((always_inline)) -> f32x16 {
        if constexpr (QK8) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, q, c, 0, 0, 0, 0, 0, 0);
        else return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q, c, 0, 0, 0);
    };
    // K operands of one 32-key half (all k-steps), then its MFMAs
    auto k_operands = [&](int slot, int half, qop (&a)[SK]) __attribute__((always_inline)) {
        const unsigned char* Ks = Kbuf + slot * K_BYTES;
#pragma unroll
        for (int ks = 0; ks < SK; ++ks) a[ks] = k_operand(Ks, 32 * half + n, ks);
    };
    auto qk_mfma = [&](const qop (&a)[SK], f32x16 (&s)[QB]) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < SK; ++ks)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[qb] = qk_step(a[ks], qreg[qb][ks], s[qb]);
    };
    auto qk_half = [&](int slot, int half, f32x16 (&s)[QB]) __attribute__((always_inline)) {
        qop a[SK];
        k_operands(slot, half, a);
        qk_mfma(a, s);
    };

    f32x16 oacc[MO][QB];
    // reference max per query, in the log2 domain (logit * log2(e)): the
    // logits of key tiles with different scales compare only after scaling
    float mref[QB];
    float nb[QB];                             // -mref
    float lsum[QB];                           // this lane's partial row sums
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int i = 0; i < MO; ++i) oacc[i][qb] = f32x16{};
        mref[qb] = -INFINITY;
        nb[qb] = 0.f;
        lsum[qb] = 0.f;
    }
    bool need_ref = true;                     // some row of the wave has no reference yet
    // log2-domain scale of the raw dot products of key tile e: scale *
    // log2(e), times the query's and the key tile's scales for e4m3 codes
    auto tile_c2 = [&](const TileEnt& e, float (&c2t)[QB]) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) c2t[qb] = QK8 ? c2q[qb] * e.ks : c2q[qb];
    };
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    // keys at or past `lim` are hidden (-inf) in one 32-key half starting at kb0
    auto apply_mask = [&](f32x16 (&s)[QB], int kb0, const int (&lim)[QB]) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kb0 + 8 * (r >> 2) + 4 * g + (r & 3);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                if (key >= lim[qb]) s[qb][r] = -INFINITY;
        }
    };
    // row max of one 32-key half (both query blocks), across the lane pair
    auto half_max = [&](const f32x16 (&s)[QB], float (&mt)[QB]) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float ma = max3(s[qb][0], s[qb][1], s[qb][2]);
            float mb = max3(s[qb][3], s[qb][4], s[qb][5]);
            ma = max3(ma, s[qb][6], s[qb][7]);
            mb = max3(mb, s[qb][8], s[qb][9]);
            ma = max3(ma, s[qb][10], s[qb][11]);
            mb = max3(mb, s[qb][12], s[qb][13]);
            ma = max3(ma, s[qb][14], s[qb][15]);
            const float m = __builtin_fmaxf(ma, mb);
            mt[qb] = __builtin_fmaxf(m, swap_halves(m));
        }
    };
    // rows without a reference yet take this half's max as their reference
    auto set_reference = [&](const f32x16 (&s)[QB], const float (&c2t)[QB]) __attribute__((always_inline)) {
        float mt[QB];
        half_max(s, mt);
        bool unset = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            mref[qb] = (mref[qb] == -INFINITY) ? mt[qb] * c2t[qb] : mref[qb];
            nb[qb] = (mref[qb] == -INFINITY) ? 0.f : -mref[qb];
            unset |= mref[qb] == -INFINITY;
        }
        need_ref = __builtin_amdgcn_ballot_w64(unset) != 0;
    };
    // weights of one key pair (pair i of 16-key chunk c of a half, MFMA k
    // order) of query block qb, packed to bf16; the pair adds to the row sum
    auto exp_pair = [&](const f32x16 (&s)[QB], int c, int qb, int i, u32x4 (&w)[QB], const float (&c2t)[QB])
                        __attribute__((always_inline)) {
        const int r = 8 * c + 2 * i;
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][r], c2t[qb], nb[qb]));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][r + 1], c2t[qb], nb[qb]));
        const uint32_t pr = f32x2_to_bf16x2(e0, e1);
        w[qb][i] = pr;
        lsum[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pr), ones, lsum[qb], false);
    };
    // weights of 16-key chunk c (0 or 1) of a half: 4 bf16 pairs per query block
    auto exp_chunk = [&](const f32x16 (&s)[QB], int c, u32x4 (&w)[QB], const float (&c2t)[QB]) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int i = 0; i < 4; ++i) exp_pair(s, c, qb, i, w, c2t);
    };
    // O^T += V^T P^T for the 16-key chunk ks (0..3) of the tile
    // V^T operands of the 16-key chunk ks (all d blocks), then its MFMAs
    auto v_operands = [&](int slot, int ks, bf16x8 (&a)[MO]) __attribute__((always_inline)) {
        const unsigned char* Vs = Vbuf + slot * V_BYTES;
        const int chunk = 2 * ks + g;
#pragma unroll
        for (int mb = 0; mb < MO; ++mb) {
            const int d = 32 * mb + n;
            a[mb] = *reinterpret_cast<const bf16x8*>(Vs + v_addr(d, chunk));
        }
    };
    auto pv_mfma = [&](const bf16x8 (&a)[MO], const u32x4 (&w)[QB]) __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < MO; ++mb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                oacc[mb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], __builtin_bit_cast(bf16x8, w[qb]),
                                                                      oacc[mb][qb], 0, 0, 0);
    };
    auto pv_chunk = [&](int slot, int ks, const u32x4 (&w)[QB]) __attribute__((always_inline)) {
        bf16x8 a[MO];
        v_operands(slot, ks, a);
        pv_mfma(a, w);
    };

    // ---- walk the key tiles -----------------------------------------------
    // mode 0: weights against the per-row reference (the fast path)
    // mode 1: exact row maxima only (QK, no weights); they become the references
    //
    // Tiles that need no mask run a branch-free, software-ordered body (in a
    // dense walk a wave whose rows all end before such a tile takes it with
    // zero weights; in a block-sparse walk a wave skips the tiles it does not
    // own); tiles that set a wave's references and masked tiles run a
    // general body.  The two bodies sit in separate loops, so the
    // accumulators only flow from one loop into the next.
    auto walk = [&](auto mode_tag) __attribute__((always_inline)) {
        constexpr int MODE = decltype(mode_tag)::value;
        reset_walk();
        // tile j of the walk lives in ring slot j % RING; at the start of an
        // iteration tiles j .. j+AHEAD-1 are in LDS
        TileEnt e0 = next_tile();
        TileEnt e1 = next_tile();
        TileEnt e2 = AHEAD == 2 ? next_tile() : TileEnt{-1, 0, 1.f};
        const bool pre = first_tile_preloaded && e0.tile == 0;
        first_tile_preloaded = false;
        if (e0.tile >= 0) {
            if (!pre) load_k(e0.tile * KT, 0);
            if constexpr (MODE == 0) {
                if (!pre) load_v(e0.tile * KT);
                store_v(0);
            }
        }
        if constexpr (AHEAD == 2) {
            if (e1.tile >= 0) {
                load_k(e1.tile * KT, 1);
                if constexpr (MODE == 0) {
                    load_v(e1.tile * KT);
                    store_v(1);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): K bytes are in LDS
        __syncthreads();

        int j = 0;
        auto fast = [&](const TileEnt& e, int idx) __attribute__((always_inline)) -> bool {
            // (in a dense walk a tile past some waves' key limits also runs the
            // branch-free body there: those waves shift their logits to -inf, so
            // their weights are zero.  In a block-sparse walk a wave's first owned tile need not be the
            // walk's first, so a tile that a wave owns while its rows have no
            // reference max yet takes the general body, which sets it.  In a
            // dense walk a row that sees any tile of its key range sees the
            // range's first tile, so every reference is set at j = 0)
            if constexpr (SPARSE) {
                if (need_ref && mine(e)) return false;
            }
            return idx > 0 && e.tile * KT + KT <= wg_kmin;
        };

        // One tile: e's K and V^T sit in LDS slot `slot`; the V of tile nv (if
        // any) is loaded now and staged into slot `vslot`.
        auto body = [&](auto fast_tag, const TileEnt& e, int slot, const TileEnt& nv, int vslot)
                        __attribute__((always_inline)) {
            constexpr bool FAST = decltype(fast_tag)::value;
            if constexpr (MODE == 0) {
                // the branch-free body always stages a V tile into the idle
                // slot; with no next tile it re-stages its own (never read)
                if (FAST || nv.tile >= 0) load_v((nv.tile >= 0 ? nv.tile : e.tile) * KT);
            }
            const int kb = e.tile * KT;
            f32x16 s0[QB], s1[QB];
            float c2t[QB];
            tile_c2(e, c2t);
            if constexpr (MODE == 0 && FAST) {
                // Software-ordered body: slot m issues MFMA m and a fixed share of
                // independent work, and a scheduling fence closes the slot, so the
                // single wave of the SIMD keeps its matrix unit fed while it
                // computes the weights.  The QK MFMAs run block by block, so the
                // weights of a 32x32 S^T block start as soon as it is complete;
                // the weight pairs are spread over the slots (WeightSlots), each
                // in three stages (scale+shift, exp2, pack+row sum) in three
                // consecutive slots.  Operand reads run a phase ahead; the next V
                // tile is staged under the last PV chunk.
                const unsigned char* Ks = Kbuf + slot * K_BYTES;
                const unsigned char* Vs = Vbuf + slot * V_BYTES;
                auto kread = [&](int half, int ks) __attribute__((always_inline)) -> qop {
                    return k_operand(Ks, 32 * half + n, ks);
                };
                auto vread = [&](int ks, int mb) __attribute__((always_inline)) -> bf16x8 {
                    return *reinterpret_cast<const bf16x8*>(Vs + v_addr(32 * mb + n, 2 * ks + g));
                };
                // MFMA operands read from LDS are handed to the MFMA from AGPRs
                // (the loads then write AGPRs), which leaves the VGPRs to O, S and
                // the weights
                auto in_agpr = [](auto x) __attribute__((always_inline)) {
                    asm("" : "+a"(x));
                    return x;
                };
                constexpr int L = QB * SK;                 // QK slots per half
                constexpr int NP = QB * MO;                // PV slots per 16-key chunk
                // (e4m3 QK chains are one quarter as long, so the first weights
                // have fewer slots before their PV MFMA: up to 4 starts a slot)
                constexpr WeightSlots<SK, NP, QK8 ? 4 : (D == 128 ? 1 : 2), QB> WS{};
                static_assert(WS.valid(), "weight pairs scheduled in time");
                const bool own = mine(e);
                float nbt[QB];
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) nbt[qb] = own ? nb[qb] : -INFINITY;
                u32x4 w[4][QB];                            // [chunk][qb]
                float xs[WS.NPAIR][2];                     // weight-pair stage values
                qop ka[SK], kb1[SK];
                bf16x8 va[4][MO];
#pragma unroll
                for (int ks = 0; ks < SK; ++ks) ka[ks] = kread(0, ks);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) s0[qb] = s1[qb] = f32x16{};
                static_for<2 * L + 4 * NP>([&](auto mc) __attribute__((always_inline)) {
                    constexpr int m = decltype(mc)::value;
                    if constexpr (m < 2 * L) {
                        // QK chains: S^T block (h, qb) in slots (QB*h+qb)*SK .. +SK-1
                        constexpr int chain = m / SK, ks = m % SK, h = chain / QB, qb = chain % QB;
                        if constexpr (h == 0) s0[qb] = qk_step(in_agpr(ka[ks]), qreg[qb][ks], s0[qb]);
                        else s1[qb] = qk_step(in_agpr(kb1[ks]), qreg[qb][ks], s1[qb]);
                        // K operands of h1 during QK(h0), V operands of chunk 0 (two
                        // query blocks: chunks 0, 1) during QK(h1)
                        if constexpr (QB == 2) {
                            if constexpr (m < L && (m & 1) == 1) kb1[m >> 1] = kread(1, m >> 1);
                        } else {
                            if constexpr (m < L) kb1[m] = kread(1, m);
                        }
                        if constexpr (m >= L) {
                            constexpr int NE = QB * MO;
                            static_for<NE>([&](auto ec) __attribute__((always_inline)) {
                                constexpr int e = decltype(ec)::value;
                                if constexpr ((e * L) / NE == m - L) va[e / MO][e % MO] = vread(e / MO, e % MO);
                            });
                        }
                    } else {
                        // PV chunks 0..3 | V operands of the later chunks | staging of the next V tile
                        constexpr int t = m - 2 * L, c = t / NP, mb = (t % NP) / QB, qb = t % QB;
                        oacc[mb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            in_agpr(va[c][mb]), __builtin_bit_cast(bf16x8, w[c][qb]), oacc[mb][qb], 0, 0, 0);
                        if constexpr (QB == 2) {
                            // (chunks 2, 3 during chunk 0)
                            if constexpr (t < NP) {
                                static_for<2 * MO>([&](auto ec) __attribute__((always_inline)) {
                                    constexpr int e = decltype(ec)::value;
                                    if constexpr ((e * NP) / (2 * MO) == t) va[2 + e / MO][e % MO] = vread(2 + e / MO, e % MO);
                                });
                            }
                        } else {
                            // (chunk c + 1 during chunk c, one operand a slot)
                            if constexpr (c < 3) va[c + 1][t % NP] = vread(c + 1, t % NP);
                        }
                        if constexpr (c == 3) {
                            static_for<4 * V_PER_T>([&](auto ec) __attribute__((always_inline)) {
                                constexpr int ev = decltype(ec)::value;
                                if constexpr ((ev * NP) / (4 * V_PER_T) == t - 3 * NP) store_v_piece(vslot, ev >> 2, ev & 3);
                            });
                        }
                    }
                    // weight pipeline: stage 3, stage 2, stage 1 (oldest first)
                    static_for<WS.NPAIR>([&](auto ic) __attribute__((always_inline)) {
                        constexpr int i = decltype(ic)::value;
                        constexpr int h = WS.half_of(i), qb = WS.qb_of(i), c = (i >> 2) & 1, ii = i & 3;
                        constexpr int r = 8 * c + 2 * ii;
                        constexpr int at = WS.at[i];
                        if constexpr (at + 2 == m) {
                            const uint32_t pr = f32x2_to_bf16x2(xs[i][0], xs[i][1]);
                            w[2 * h + c][qb][ii] = pr;
                            lsum[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pr), ones, lsum[qb], false);
                        }
                        if constexpr (at + 1 == m) {
                            xs[i][0] = __builtin_amdgcn_exp2f(xs[i][0]);
                            xs[i][1] = __builtin_amdgcn_exp2f(xs[i][1]);
                        }
                        if constexpr (at == m) {
                            if constexpr (h == 0) {
                                xs[i][0] = __builtin_fmaf(s0[qb][r], c2t[qb], nbt[qb]);
                                xs[i][1] = __builtin_fmaf(s0[qb][r + 1], c2t[qb], nbt[qb]);
                            } else {
                                xs[i][0] = __builtin_fmaf(s1[qb][r], c2t[qb], nbt[qb]);
                                xs[i][1] = __builtin_fmaf(s1[qb][r + 1], c2t[qb], nbt[qb]);
                            }
                        }
                    });
                    __builtin_amdgcn_sched_barrier(0);
                });
            } else {
                // a tile outside this wave's own list is computed fully masked
                const bool own = mine(e);
                int lim[QB];
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) lim[qb] = own ? klim[qb] : -1;
                const bool need_mask = kb + KT > (own ? w_kmin : -1);
                if constexpr (MODE == 0) {
                    u32x4 w00[QB], w01[QB], w10[QB], w11[QB];
                    qk_half(slot, 0, s0);
                    if (need_mask) apply_mask(s0, kb, lim);
                    if (need_ref) set_reference(s0, c2t);
                    qk_half(slot, 1, s1);
                    if (need_mask) apply_mask(s1, kb + 32, lim);
                    if (need_ref) set_reference(s1, c2t);
                    exp_chunk(s0, 0, w00, c2t);
                    exp_chunk(s0, 1, w01, c2t);
                    exp_chunk(s1, 0, w10, c2t);
                    exp_chunk(s1, 1, w11, c2t);
                    pv_chunk(slot, 0, w00);
                    pv_chunk(slot, 1, w01);
                    pv_chunk(slot, 2, w10);
                    pv_chunk(slot, 3, w11);
                } else {
                    float mt[QB];
                    qk_half(slot, 0, s0);
                    if (need_mask) apply_mask(s0, kb, lim);
                    half_max(s0, mt);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) mref[qb] = __builtin_fmaxf(mref[qb], mt[qb] * c2t[qb]);
                    qk_half(slot, 1, s1);
                    if (need_mask) apply_mask(s1, kb + 32, lim);
                    half_max(s1, mt);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) mref[qb] = __builtin_fmaxf(mref[qb], mt[qb] * c2t[qb]);
                }
            }
            if constexpr (MODE == 0 && !FAST) {
                if (nv.tile >= 0) store_v(vslot);
            }
        };
        // the DMA'd K tiles are in LDS and every wave is past its reads of the
        // slots that the next loads overwrite
        auto tile_barrier = [&]() __attribute__((always_inline)) {
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
            __syncthreads();
        };
        // Wide block-sparse walk: tile pairs once no wave of the workgroup
        // lacks a reference (a workgroup-uniform flag, from the words the
        // waves post at each single tile's barrier) and neither tile needs a
        // mask; a wave that does not own a tile of the pair takes it with
        // zero weights
        constexpr bool SPAIRS = SPARSE && WIDE && MODE == 0;
        bool all_ref = false;
        auto pair_ok = [&]() __attribute__((always_inline)) -> bool {
            return SPAIRS && all_ref && e1.tile >= 0 && j > 0 && e0.tile * KT + KT <= wg_kmin &&
                   e1.tile * KT + KT <= wg_kmin;
        };
        // one tile per barrier; the tile AHEAD places on is loaded meanwhile
        auto single = [&](auto fast_tag) __attribute__((always_inline)) {
            const TileEnt nx = AHEAD == 2 ? e2 : e1;
            if (nx.tile >= 0) load_k(nx.tile * KT, (j + AHEAD) % RING);
            if constexpr (decltype(fast_tag)::value == 2) {
                // Block-sparse, a tile outside this wave's own list: it adds
                // nothing to the wave's rows (their weights there are zero), so
                // the wave only stages its share of the next V tile, and the
                // SIMD's matrix unit goes to the other wave on it (of the other
                // workgroup)
                if constexpr (MODE == 0) {
                    if (nx.tile >= 0) {
                        load_v(nx.tile * KT);
                        store_v((j + AHEAD) % RING);
                    }
                }
            } else {
                body(BoolC<decltype(fast_tag)::value == 1>{}, e0, j % RING, nx, (j + AHEAD) % RING);
            }
            if constexpr (SPAIRS) {
                if (!all_ref && lane == 0) ref_words[j & 1][wave] = need_ref ? 1 : 0;
            }
            tile_barrier();
            if constexpr (SPAIRS) {
                if (!all_ref) {
                    int any = 0;
#pragma unroll
                    for (int w = 0; w < NW; ++w) any |= ref_words[j & 1][w];
                    all_ref = __builtin_amdgcn_readfirstlane(any) == 0;
                }
            }
            e0 = e1;
            if constexpr (AHEAD == 2) {
                e1 = e2;
                e2 = next_tile();
            } else {
                e1 = next_tile();
            }
            ++j;
        };
        // two branch-free tiles per barrier (wide walks): the two after them are
        // loaded meanwhile
        auto pair = [&]() __attribute__((always_inline)) {
            const TileEnt e3 = next_tile();
            if (e2.tile >= 0) load_k(e2.tile * KT, (j + 2) & 3);
            if (e3.tile >= 0) load_k(e3.tile * KT, (j + 3) & 3);
            body(BoolC<true>{}, e0, j & 3, e2, (j + 2) & 3);
            body(BoolC<true>{}, e1, (j + 1) & 3, e3, (j + 3) & 3);
            tile_barrier();
            e0 = e2;
            e1 = e3;
            e2 = next_tile();
            j += 2;
        };
        while (e0.tile >= 0) {
            if constexpr (MODE == 0 && !SPARSE) {
                // (the pair decision is workgroup-uniform in a dense walk)
                while (e1.tile >= 0 && fast(e0, j) && fast(e1, j + 1)) pair();
                if (e0.tile >= 0) single(IntC<0>{});
            } else {
                // (block-sparse: three loops, one per body, one barrier per tile
                // in each, so the waves of a workgroup may sit in different loops;
                // a wide walk leaves them all, at the same tile, for tile pairs)
                if constexpr (SPAIRS) {
                    while (pair_ok()) pair();
                }
                if constexpr (SPARSE) {
                    while (e0.tile >= 0 && !mine(e0) && !pair_ok()) single(IntC<2>{});
                }
                if constexpr (MODE == 0) {
                    while (e0.tile >= 0 && (!SPARSE || mine(e0)) && fast(e0, j) && !pair_ok()) single(IntC<1>{});
                }
                while (e0.tile >= 0 && (!SPARSE || mine(e0)) && (MODE != 0 || !fast(e0, j)) && !pair_ok())
                    single(IntC<0>{});
            }
        }
    };

    walk(IntC<0>{});
    // a row sum above 2^100 (or inf/nan) means logits far above the row's
    // reference: recompute against the exact row maxima (rare; workgroup-wide).
    // So does an accumulator that is no longer finite (weights up to 2^100
    // times large values of v).  The tests look at exponent bits: the kernel
    // is built without NaN semantics, so float comparisons cannot see a NaN.
    {
        bool bad = false;
        uint32_t obits = 0u;   // largest |O| bit pattern of the lane
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int mb = 0; mb < MO; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) obits = max(obits, __float_as_uint(oacc[mb][qb][r]) & 0x7fffffffu);
        bad |= obits >= 0x7f800000u;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float ltot = lsum[qb] + swap_halves(lsum[qb]);
            // a sum out of range, or a row that saw keys only in branch-free
            // tiles before it had a reference, needs the exact recompute
            bad |= (__float_as_uint(ltot) & 0x7fffffffu) > __float_as_uint(kSumLimit) ||
                   (mref[qb] == -INFINITY && ltot > 0.f);
        }
        // one flag per wave, in words no walk overwrites: one barrier
        int* flags = wg_words + 2 * NW;
        const bool wave_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
        if (lane == 0) flags[wave] = wave_bad ? 1 : 0;
        __syncthreads();
        int again = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) again |= flags[w];
        again = __builtin_amdgcn_readfirstlane(again);
        if (again) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) mref[qb] = -INFINITY;
            walk(IntC<1>{});
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                nb[qb] = (mref[qb] == -INFINITY) ? 0.f : -mref[qb];
                lsum[qb] = 0.f;
#pragma unroll
                for (int i = 0; i < MO; ++i) oacc[i][qb] = f32x16{};
            }
            need_ref = false;
            walk(IntC<0>{});
        }
    }

    // ---- epilogue --------------------------------------------------------
    unsigned char* ob = reinterpret_cast<unsigned char*>(p.o);
    const bool partial = n_sp > 1;   // write this split's normalised O and LSE (fp32) for the merge
    // partial rows are numbered over the split items only: (b, h, row) flattened,
    // from the first row of item split_from (part_first), part_rows per split
    const int64_t part_row0 = (int64_t)split * p.part_rows + (int64_t)(b * p.H + h) * p.n_rows - p.part_first;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float ltot = lsum[qb] + swap_halves(lsum[qb]);
        const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
        if (!row_valid[qb]) continue;
        if (partial) {
            float* po = p.part_o + (part_row0 + my_row[qb]) * D;
#pragma unroll
            for (int mb = 0; mb < MO; ++mb)
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    *reinterpret_cast<float4*>(po + 32 * mb + 8 * a + 4 * g) =
                        make_float4(oacc[mb][qb][4 * a + 0] * inv, oacc[mb][qb][4 * a + 1] * inv,
                                    oacc[mb][qb][4 * a + 2] * inv, oacc[mb][qb][4 * a + 3] * inv);
        } else {
            const int orow = out_row_of(p, my_row[qb]);
#pragma unroll
            for (int mb = 0; mb < MO; ++mb) {
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int d0 = 32 * mb + 8 * a + 4 * g;
                    const float x0 = oacc[mb][qb][4 * a + 0] * inv, x1 = oacc[mb][qb][4 * a + 1] * inv;
                    const float x2 = oacc[mb][qb][4 * a + 2] * inv, x3 = oacc[mb][qb][4 * a + 3] * inv;
                    const int64_t e = b * p.o_sb + h * p.o_sh + (int64_t)orow * p.o_st + d0;
                    if constexpr (OUT_BF16) {
                        *reinterpret_cast<u32x2*>(ob + e * 2) = u32x2{f32x2_to_bf16x2(x0, x1), f32x2_to_bf16x2(x2, x3)};
                    } else {
                        *reinterpret_cast<float4*>(ob + e * 4) = make_float4(x0, x1, x2, x3);
                    }
                }
            }
        }
        if (g == 0) {
            const float l = ltot > 0.f ? mref[qb] * 0.69314718055994531f + __logf(ltot) : -INFINITY;
            if (partial) p.part_lse[part_row0 + my_row[qb]] = l;
            else if (p.lse) p.lse[(int64_t)(b * p.H + h) * p.n_rows + my_row[qb]] = l;
        }
    }
}

// Combination of the key splits of one launch: per row of a split item, O =
// sum_s w_s O_s / sum_s w_s and LSE = M + log(sum_s w_s) with w_s =
// exp(LSE_s - M), M the largest LSE_s (a split in which the row sees no key
// has LSE_s = -inf and weight 0).  One thread per 4 output columns of a row;
// the threads cover items [split_from, items) only, rows_per_item rows each.
// NS = n_splits, so every load of a thread is issued before the first is used.
template <bool OUT_BF16, int NS>
__global__ __launch_bounds__(256) void split_merge_kernel(const AttnParams p, int D, int rows_per_item) {
    const int cpr = D / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t items = (int64_t)p.n_qtiles * p.B * p.H;
    if (idx >= (items - p.split_from) * rows_per_item * cpr) return;
    const int c = (int)(idx % cpr);
    const int64_t t = idx / cpr;
    const int item = p.split_from + (int)(t / rows_per_item);
    const int qtile = item % p.n_qtiles;
    const int bh = item / p.n_qtiles;
    const int row = qtile * rows_per_item + (int)(t % rows_per_item);
    if (row >= p.n_rows) return;
    const int b = bh / p.H, h = bh - b * p.H;
    const int64_t rr = (int64_t)bh * p.n_rows + row;
    const int64_t plane = p.part_rows;
    const int64_t pr = rr - p.part_first;   // this row among the split items' rows
    float l[NS];
    float4 o[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        l[s] = p.part_lse[s * plane + pr];
        o[s] = *reinterpret_cast<const float4*>(p.part_o + (s * plane + pr) * D + 4 * c);
    }
    float m = -INFINITY;
#pragma unroll
    for (int s = 0; s < NS; ++s) m = __builtin_fmaxf(m, l[s]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float wsum = 0.f;
    if (m != -INFINITY) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const float w = __expf(l[s] - m);
            acc.x += w * o[s].x;
            acc.y += w * o[s].y;
            acc.z += w * o[s].z;
            acc.w += w * o[s].w;
            wsum += w;
        }
    }
    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    const int64_t e = b * p.o_sb + h * p.o_sh + (int64_t)out_row_of(p, row) * p.o_st + 4 * c;
    if constexpr (OUT_BF16) {
        *reinterpret_cast<u32x2*>(reinterpret_cast<unsigned char*>(p.o) + e * 2) =
            u32x2{f32x2_to_bf16x2(acc.x * inv, acc.y * inv), f32x2_to_bf16x2(acc.z * inv, acc.w * inv)};
    } else {
        *reinterpret_cast<float4*>(reinterpret_cast<unsigned char*>(p.o) + e * 4) =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
    if (p.lse && c == 0) p.lse[rr] = wsum > 0.f ? m + __logf(wsum) : -INFINITY;
}

template <bool OUT_BF16>
hipError_t launch_merge(const AttnParams& p, int D, int rows_per_item, unsigned blocks, hipStream_t s) {
    static_assert(kMaxSplits == 8, "one instantiation per split count");
    switch (p.n_splits) {
    case 2: hipLaunchKernelGGL((split_merge_kernel<OUT_BF16, 2>), dim3(blocks), dim3(256), 0, s, p, D, rows_per_item); break;
    case 3: hipLaunchKernelGGL((split_merge_kernel<OUT_BF16, 3>), dim3(blocks), dim3(256), 0, s, p, D, rows_per_item); break;
    case 4: hipLaunchKernelGGL((split_merge_kernel<OUT_BF16, 4>), dim3(blocks), dim3(256), 0, s, p, D, rows_per_item); break;
    case 5: hipLaunchKernelGGL((split_merge_kernel<OUT_BF16, 5>), dim3(blocks), dim3(256), 0, s, p, D, rows_per_item); break;
    case 6: hipLaunchKernelGGL((split_merge_kernel<OUT_BF16, 6>), dim3(blocks), dim3(256), 0, s, p, D, rows_per_item); break;
    case 7: hipLaunchKernelGGL((split_merge_kernel<OUT_BF16, 7>), dim3(blocks), dim3(256), 0, s, p, D, rows_per_item); break;
    case 8: hipLaunchKernelGGL((split_merge_kernel<OUT_BF16, 8>), dim3(blocks), dim3(256), 0, s, p, D, rows_per_item); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Workgroups of one instantiation that a compute unit holds at once (1 when
// the runtime cannot say).
template <int D, bool OB, bool SP, bool QK8, int QB, bool WIDE = !SP, bool RESTORE = false>
int resident_wgs() {
    static const int n = [] {
        int k = 0;
        const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &k, attn_kernel<D, OB, SP, QK8, QB, WIDE, RESTORE>, waves_per_wg<SP, QB>() * 64, 0);
        if (e != hipSuccess) (void)hipGetLastError();
        return e == hipSuccess && k > 0 ? k : 1;
    }();
    return n;
}

// The host bounds split_from + (items - split_from) * n_splits below 2^31 and
// sets split_from = items when n_splits == 1.  RESTORE: p.rs_wgs
// reconstruction workgroups follow the attention's (no key splits).
template <int D, bool OB, bool SP, bool QK8, int QB, bool WIDE = !SP, bool RESTORE = false>
hipError_t launch_one(const AttnParams& p, hipStream_t s) {
    const int items = p.n_qtiles * p.B * p.H;
    const int grid = p.split_from + (items - p.split_from) * p.n_splits + (RESTORE ? p.rs_wgs : 0);
    hipLaunchKernelGGL((attn_kernel<D, OB, SP, QK8, QB, WIDE, RESTORE>), dim3(grid), dim3(waves_per_wg<SP, QB>() * 64), 0,
                       s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.split_from == items) return e;
    constexpr int QT = rows_per_wg<SP, QB>();
    const int64_t threads = (int64_t)(items - p.split_from) * QT * (D / 4);
    return launch_merge<OB>(p, D, QT, (unsigned)((threads + 255) / 256), s);
}

}  // namespace
}  // namespace varattn
