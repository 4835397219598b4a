// Block-causal next-scale attention, bf16 in / fp32 accumulate, for gfx950.
//
// Computes, for every query row of the call, O = softmax(scale * q K^T) V over
// the keys the row may see: all keys of its own and earlier scales ("SparVAR:
// Exploring Sparsity in Visual AutoRegressive Modeling for Training-Free
// Acceleration", abstract: each step attends to all tokens of the historical
// scales; "ARVAR: Accelerating Visual Autoregressive Model via Attention
// Retrospect", Background & Motivation: a whole grid per step with a KV
// cache).  A key u is visible to token t iff u < end of t's scale, so
// visibility is one key limit per query.  The block-sparse variant walks the
// kept key tiles of its query tile instead of all of them ("SparVAR ...",
// abstract: block-wise sparse attention); the optional q_index fuses the
// gather of pruned queries ("ARVAR ...", Key Design 2).
//
// Design (one workgroup = NW waves = 32*NW query rows of one (batch, head)):
//  * Each wave owns 32 queries.  It computes S^T = K Q^T with
//    v_mfma_f32_32x32x16_bf16 (keys on M, queries on N), so every lane holds
//    16 logits of ONE query and lane l^32 holds the other 16 of a 32-key
//    block: the row max / row sum need one cross-lane exchange per tile.
//  * The same registers, converted to bf16, are directly the B operand of
//    O^T += V^T P^T (d on M, queries on N, keys on K): the MFMA's k-order is
//    matched by permuting the keys of V^T inside LDS, so P never moves.
//  * Q stays in registers for the whole key loop (B operand of S^T).
//  * K (row-major, 16-byte chunks XOR-swizzled) and V^T (transposed through
//    registers, keys permuted, 16-byte chunks XOR-swizzled) are staged in a
//    double-buffered LDS ring: one barrier per 64-key tile, the next tile's
//    global loads in flight during the current tile's MFMAs.
//  * Online softmax in the log2 domain (scale*log2(e) folded into one FMA
//    before v_exp_f32), with lazy rescaling: the running reference max only
//    moves when some row's max grows by more than 2^8, so O is rescaled
//    rarely.
//  * Workgroup ids are remapped so that the query tiles of one (batch, head)
//    run on the same XCD and share its L2 for K and V.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace varattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int KT = 64;                 // keys per tile (= sparse tile width)
constexpr float kRescaleLog2 = 8.0f;   // lazy-rescale threshold (log2 units)

__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
    // The dispatcher places workgroup i on XCD i % 8.  Give each XCD a
    // contiguous range of work items so neighbours share an L2.
    const int q = nwg >> 3, r = nwg & 7;
    const int x = wg & 7, j = wg >> 3;
    return x * q + (x < r ? x : r) + j;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
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

// K tile: row r (key), 16-byte chunk c -> swizzled chunk.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
    if constexpr (D == 128) return r & 15;        // 256-byte rows
    else return (r >> 1) & 7;                     // 128-byte rows
}
// V^T tile: 128-byte rows (64 keys), row = d.
__device__ __forceinline__ int v_swz(int d) { return (d >> 1) & 7; }

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
    const __bf16 x = (__bf16)a, y = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

template <int D, int NW, bool OUT_BF16, bool SPARSE>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(const AttnParams p) {
    constexpr int NT = NW * 64;
    constexpr int QT = NW * 32;
    constexpr int KCH = D / 8;                 // 16-byte chunks per K row
    constexpr int K_BYTES = KT * D * 2;
    constexpr int V_BYTES = KT * D * 2;
    constexpr int BUF = K_BYTES + V_BYTES;
    constexpr int K_PER_T = KT * KCH / NT;     // 16-byte K chunks per thread
    constexpr int V_UNITS = (KT / 4) * (D / 4);
    constexpr int V_PER_T = V_UNITS / NT;      // 4x4 V blocks per thread
    static_assert(K_PER_T * NT == KT * KCH, "K tile split");
    static_assert(V_PER_T * NT == V_UNITS, "V tile split");
    constexpr int SK = D / 16;                 // k-steps of S^T = K Q^T
    constexpr int MO = D / 32;                 // 32-row blocks of O^T

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 5;      // lane half
    const int n = lane & 31;      // query column inside the wave

    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int qtile = item % p.n_qtiles;
    const int bh = item / p.n_qtiles;
    const int b = bh / p.H;
    const int h = bh - b * p.H;

    // ---- this lane's query row ------------------------------------------
    const int my_row = qtile * QT + wave * 32 + n;
    const bool row_valid = my_row < p.n_rows;
    const int row_c = row_valid ? my_row : (p.n_rows - 1);
    int pos = p.q_index ? p.q_index[row_c] : row_c;
    pos = pos < 0 ? 0 : (pos >= p.n_q ? p.n_q - 1 : pos);
    const int tok = p.q_first + pos;
    int klim = p.kv_len;
    if (!p.step_mode) {
#pragma unroll
        for (int s = VAR_MAX_SCALES - 1; s >= 0; --s)
            if (s < p.num_scales && tok < p.scale_end[s]) klim = p.scale_end[s];
    }
    const int w_kmin = wave_min_i(klim);
    const int w_kmax = wave_max_i(klim);

    const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)pos * p.q_st;
    bf16x8 qreg[SK];
#pragma unroll
    for (int ks = 0; ks < SK; ++ks)
        qreg[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 16 * ks + 8 * g));

    // ---- key-tile list ------------------------------------------------------
    int n_tiles, list_begin = 0;
    if constexpr (SPARSE) {
        list_begin = p.row_ptr[qtile];
        n_tiles = p.row_ptr[qtile + 1] - list_begin;
    } else {
        int* red = reinterpret_cast<int*>(smem);
        if (lane == 0) red[wave] = w_kmax;
        __syncthreads();
        int m = red[0];
#pragma unroll
        for (int i = 1; i < NW; ++i) m = max(m, red[i]);
        __syncthreads();
        n_tiles = (m + KT - 1) / KT;
    }

    const __bf16* kp = reinterpret_cast<const __bf16*>(p.k) + b * p.k_sb + h * p.k_sh;
    const __bf16* vp = reinterpret_cast<const __bf16*>(p.v) + b * p.v_sb + h * p.v_sh;
    const int kv_last = p.kv_len - 1;

    u32x4 kreg[K_PER_T];
    u32x2 vreg[V_PER_T][4];

    auto tile_base = [&](int it) __attribute__((always_inline)) -> int {
        if constexpr (SPARSE) {
            // a column outside [0, n_kt) cannot come from the mask builder; clamp so loads stay in bounds
            const int c = p.col_idx[list_begin + it];
            return min(max(c, 0), (p.kv_len - 1) / KT) * KT;
        } else {
            return it * KT;
        }
    };
    auto load_tile = [&](int kbase) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < K_PER_T; ++j) {
            const int c = tid + NT * j;
            const int r = c / KCH, col = c % KCH;
            const int key = min(kbase + r, kv_last);
            kreg[j] = *reinterpret_cast<const u32x4*>(kp + (int64_t)key * p.k_st + col * 8);
        }
#pragma unroll
        for (int j = 0; j < V_PER_T; ++j) {
            const int u = tid + NT * j;
            const int dg = u % (D / 4), kg = u / (D / 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = min(kbase + 4 * kg + r, kv_last);
                vreg[j][r] = *reinterpret_cast<const u32x2*>(vp + (int64_t)key * p.v_st + 4 * dg);
            }
        }
    };
    auto store_tile = [&](int buf) __attribute__((always_inline)) {
        unsigned char* Ks = smem + buf * BUF;
        unsigned char* Vs = Ks + K_BYTES;
#pragma unroll
        for (int j = 0; j < K_PER_T; ++j) {
            const int c = tid + NT * j;
            const int r = c / KCH, col = c % KCH;
            *reinterpret_cast<u32x4*>(Ks + (r * KCH + (col ^ k_swz<D>(r))) * 16) = kreg[j];
        }
#pragma unroll
        for (int j = 0; j < V_PER_T; ++j) {
            const int u = tid + NT * j;
            const int dg = u % (D / 4), kg = u / (D / 4);
            // keys 4kg..4kg+3 go to position kb*16 + perm(g4)*4, perm = {0, 2, 1, 3}
            const int kb = kg >> 2, g4 = kg & 3;
            const int pg = ((g4 & 1) << 1) | (g4 >> 1);
            const int chunk = 2 * kb + (pg >> 1);
            const int half = pg & 1;
            const u32x2* a = vreg[j];
            u32x2 outv[4];
            outv[0] = u32x2{pack_lo(a[0].x, a[1].x), pack_lo(a[2].x, a[3].x)};
            outv[1] = u32x2{pack_hi(a[0].x, a[1].x), pack_hi(a[2].x, a[3].x)};
            outv[2] = u32x2{pack_lo(a[0].y, a[1].y), pack_lo(a[2].y, a[3].y)};
            outv[3] = u32x2{pack_hi(a[0].y, a[1].y), pack_hi(a[2].y, a[3].y)};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d = 4 * dg + i;
                *reinterpret_cast<u32x2*>(Vs + d * 128 + ((chunk ^ v_swz(d)) * 16) + half * 8) = outv[i];
            }
        }
    };

    f32x16 oacc[MO];
#pragma unroll
    for (int i = 0; i < MO; ++i) oacc[i] = f32x16{};
    float mref = -INFINITY;   // reference max (raw logit units)
    float lsum = 0.f;         // this lane's partial row sum
    const float c2 = p.scale_log2;

    if (n_tiles > 0) {
        load_tile(tile_base(0));
        store_tile(0);
    }
    __syncthreads();

    for (int it = 0; it < n_tiles; ++it) {
        const int cur = it & 1;
        const int kbase = tile_base(it);
        const bool has_next = it + 1 < n_tiles;
        if (has_next) load_tile(tile_base(it + 1));

        if (kbase < w_kmax) {
            const unsigned char* Ks = smem + cur * BUF;
            const unsigned char* Vs = Ks + K_BYTES;
            f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
            for (int ks = 0; ks < SK; ++ks) {
                const int chunk = 2 * ks + g;
                const int r0 = n, r1 = n + 32;
                const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(Ks + (r0 * KCH + (chunk ^ k_swz<D>(r0))) * 16);
                const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(Ks + (r1 * KCH + (chunk ^ k_swz<D>(r1))) * 16);
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[ks], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[ks], s1, 0, 0, 0);
            }
            // keys held by this lane: kbase + 8*(r/4) + 4*g + (r&3) (+32 for s1)
            if (kbase + KT > w_kmin) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kbase + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (key >= klim) s0[r] = -INFINITY;
                    if (key + 32 >= klim) s1[r] = -INFINITY;
                }
            }
            float mt = fmaxf(s0[0], s1[0]);
#pragma unroll
            for (int r = 1; r < 16; ++r) mt = fmaxf(mt, fmaxf(s0[r], s1[r]));
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const bool grow = (mt - mref) * c2 > kRescaleLog2;
            if (__builtin_amdgcn_ballot_w64(grow)) {
                const float mnew = fmaxf(mref, mt);
                const float alpha = (mref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((mref - mnew) * c2);
#pragma unroll
                for (int i = 0; i < MO; ++i) oacc[i] *= alpha;
                lsum *= alpha;
                mref = mnew;
            }
            const float nb = (mref == -INFINITY) ? 0.f : -mref * c2;
            uint32_t pk[16];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c2, nb));
                const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r + 1], c2, nb));
                const float f0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c2, nb));
                const float f1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r + 1], c2, nb));
                lsum += (e0 + e1) + (f0 + f1);
                pk[r / 2] = f32x2_to_bf16x2(e0, e1);
                pk[8 + r / 2] = f32x2_to_bf16x2(f0, f1);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                // keys 16ks..16ks+15: registers 8*(ks&1)..+7 of block ks>>1
                const u32x4 bw = u32x4{pk[4 * ks + 0], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]};
                const bf16x8 bop = __builtin_bit_cast(bf16x8, bw);
                const int chunk = 2 * ks + g;
#pragma unroll
                for (int mb = 0; mb < MO; ++mb) {
                    const int d = 32 * mb + n;
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vs + d * 128 + ((chunk ^ v_swz(d)) * 16));
                    oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, oacc[mb], 0, 0, 0);
                }
            }
        }
        if (has_next) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue --------------------------------------------------------
    const float ltot = lsum + __shfl_xor(lsum, 32);
    const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
    if (row_valid) {
        unsigned char* ob = reinterpret_cast<unsigned char*>(p.o);
#pragma unroll
        for (int mb = 0; mb < MO; ++mb) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int d0 = 32 * mb + 8 * a + 4 * g;
                const float x0 = oacc[mb][4 * a + 0] * inv, x1 = oacc[mb][4 * a + 1] * inv;
                const float x2 = oacc[mb][4 * a + 2] * inv, x3 = oacc[mb][4 * a + 3] * inv;
                const int64_t e = b * p.o_sb + h * p.o_sh + (int64_t)my_row * p.o_st + d0;
                if constexpr (OUT_BF16) {
                    *reinterpret_cast<u32x2*>(ob + e * 2) = u32x2{f32x2_to_bf16x2(x0, x1), f32x2_to_bf16x2(x2, x3)};
                } else {
                    *reinterpret_cast<float4*>(ob + e * 4) = make_float4(x0, x1, x2, x3);
                }
            }
        }
        if (p.lse && g == 0) {
            const float l = ltot > 0.f ? mref * p.scale + __logf(ltot) : -INFINITY;
            p.lse[(int64_t)(b * p.H + h) * p.n_rows + my_row] = l;
        }
    }
}

template <int D, int NW, bool OB, bool SP>
hipError_t launch_one(const AttnParams& p, hipStream_t s) {
    const int grid = p.n_qtiles * p.B * p.H;
    hipLaunchKernelGGL((attn_bf16_kernel<D, NW, OB, SP>), dim3(grid), dim3(NW * 64), 0, s, p);
    return hipGetLastError();
}

}  // namespace

int attn_bf16_rows_per_tile(int head_dim, bool sparse) {
    (void)head_dim;
    return sparse ? 64 : 128;
}

hipError_t launch_attn_bf16(const AttnParams& p, int D, bool out_bf16, bool sparse, hipStream_t s) {
    if (sparse) {
        if (D == 128) return out_bf16 ? launch_one<128, 2, true, true>(p, s) : launch_one<128, 2, false, true>(p, s);
        return out_bf16 ? launch_one<64, 2, true, true>(p, s) : launch_one<64, 2, false, true>(p, s);
    }
    if (D == 128) return out_bf16 ? launch_one<128, 4, true, false>(p, s) : launch_one<128, 4, false, false>(p, s);
    return out_bf16 ? launch_one<64, 4, true, false>(p, s) : launch_one<64, 4, false, false>(p, s);
}

}  // namespace varattn
