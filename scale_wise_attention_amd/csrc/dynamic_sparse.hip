// Per-head sparse pattern of a later step predicted from a decision scale, for gfx950.
//
// "SparVAR: Exploring Sparsity in Visual AutoRegressive Modeling for
// Training-Free Acceleration", abstract: the sparse attention pattern of the
// later high-resolution scales is predicted from a sparse decision scale, and
// the pattern of a large scale is made self-similar to it through an index
// mapping between scales.  Readings (the abstract gives no formulas):
//  * attention mass of the decision step d per (batch, head, 64-row query
//    tile r, 64-token key tile c): the sum of its attention weights;
//  * decision: per (batch, head, r) the key tiles by decreasing mass (equal
//    masses by lower c) are kept while the kept mass is below tau times the
//    row tile's total (fp32 sums in that order; the total in ascending c);
//  * index mapping to a step T >= d: a query (y, x) of scale T stands for
//    (floor(y*h_d/h_T), floor(x*w_d/w_T)) of scale d; a key of a scale j <= d
//    for itself; a key (y, x) of a scale j > d for (floor(y*h_d/h_j),
//    floor(x*w_d/w_j)) of scale d.  Tile (R, C) of step T is kept when a query
//    of R and a key of C stand for a kept decision pair.
//
// block_mass_kernel: one workgroup per (batch, head, key tile of [0, L_d)).
// Its 64 keys stay in registers as MFMA A operands; the waves stream 32-row
// query blocks (S^T = K Q^T on v_mfma_f32_32x32x16_bf16), turn the logits into
// weights with the rows' LSE from the attention of step d, and reduce each
// block's weights to one number; two blocks make a row tile.
//
// decision_kernel: one workgroup per (map, row tile): ranks by counting, then
// one lane walks the ranks in order with the fp32 running sum.
//
// mapped_mask_kernel: one workgroup per (map, query tile R of step T).  The
// decision row tiles that R's rows stand for give a set of kept decision key
// tiles; each such tile maps back to itself (its tokens of scales <= d) and,
// for every scale j in (d, T], to the preimage in grid j of its scale-d
// tokens: up to three rectangles of grid d (partial first row, full rows,
// partial last row), each with the rectangle preimage
// rows ceil(ya*h_j/h_d) .. ceil((yb+1)*h_j/h_d) - 1 (columns alike), i.e. runs
// of consecutive tokens.  The runs' key tiles are OR-ed into an LDS bitmap,
// compacted like the static tile mask, and a second launch (one workgroup per
// map) moves the lists into CSR form.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace varattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;
constexpr int kThreads = 256;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
    return v;
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void block_mass_kernel(const MassParams p) {
    constexpr int SK = D / 16;
    __shared__ float blk[kMassMaxRows / 32];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, n = lane & 31;
    const int c = blockIdx.x % p.n_kt;
    const int bh = blockIdx.x / p.n_kt;
    const int b = bh / p.H, h = bh - b * p.H;
    const __bf16* qbase = reinterpret_cast<const __bf16*>(p.q) + b * p.q_sb + h * p.q_sh;
    const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + b * p.k_sb + h * p.k_sh;
    const float* lse = p.lse + (int64_t)bh * p.n_rows;

    bf16x8 ka[2][SK];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int key = min(c * kTile + 32 * mb + n, p.kv_len - 1);
        const __bf16* kr = kbase + (int64_t)key * p.k_st;
#pragma unroll
        for (int ks = 0; ks < SK; ++ks)
            ka[mb][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kr + 16 * ks + 8 * g));
    }
    // keys of this lane's 16 registers that lie past the cache are dropped
    bool key_ok[2][16];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            key_ok[mb][r] = c * kTile + 32 * mb + 8 * (r >> 2) + 4 * g + (r & 3) < p.kv_len;

    constexpr float kLog2e = 1.4426950408889634f;
    const int n_qb = (p.n_rows + 31) / 32;
    for (int qb = wave; qb < n_qb; qb += kThreads / 64) {
        const int row = qb * 32 + n;
        const int rc = min(row, p.n_rows - 1);
        const __bf16* qr = qbase + (int64_t)rc * p.q_st;
        bf16x8 qf[SK];
#pragma unroll
        for (int ks = 0; ks < SK; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qr + 16 * ks + 8 * g));
        const float shift = row < p.n_rows ? -lse[rc] * kLog2e : -INFINITY;
        float acc_lane = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            f32x16 s = {};
#pragma unroll
            for (int ks = 0; ks < SK; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[mb][ks], qf[ks], s, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], p.scale_log2, shift));
                acc_lane += key_ok[mb][r] ? e : 0.f;
            }
        }
        const float tot = wave_sum(acc_lane);
        if (lane == 0) blk[qb] = tot;
    }
    __syncthreads();
    const int n_qt = (p.n_rows + kTile - 1) / kTile;
    for (int r = tid; r < n_qt; r += kThreads) {
        const float m = blk[2 * r] + (2 * r + 1 < n_qb ? blk[2 * r + 1] : 0.f);
        p.mass[((int64_t)bh * n_qt + r) * p.n_kt + c] = m;
    }
}

__global__ __launch_bounds__(kThreads) void decision_kernel(const DecisionParams p) {
    __shared__ float m[kDecisionMaxTiles];
    __shared__ int order[kDecisionMaxTiles];
    __shared__ unsigned char keep[kDecisionMaxTiles];
    const int tid = threadIdx.x;
    const int64_t base = (int64_t)blockIdx.x * p.n_kt;     // one (map, row tile)
    for (int c = tid; c < p.n_kt; c += kThreads) {
        m[c] = p.mass[base + c];
        order[c] = -1;
        keep[c] = 0;
    }
    __syncthreads();
    for (int c = tid; c < p.n_kt; c += kThreads) {
        const float x = m[c];
        int rank = 0;
        for (int o = 0; o < p.n_kt; ++o) {
            const float y = m[o];
            rank += (y > x || (y == x && o < c)) ? 1 : 0;
        }
        if (rank < p.n_kt) order[rank] = c;
    }
    __syncthreads();
    if (tid == 0) {
        float total = 0.f;
        for (int c = 0; c < p.n_kt; ++c) total += m[c];
        const float target = p.tau * total;
        float cum = 0.f;
        for (int k = 0; k < p.n_kt; ++k) {
            const int c = order[k];
            if (c < 0) continue;                  // only with NaN masses
            if (cum < target) keep[c] = 1;
            cum += m[c];
        }
    }
    __syncthreads();
    for (int c = tid; c < p.n_kt; c += kThreads) p.kept[base + c] = keep[c];
}

// Set the bits of key tiles [t0, t1] (all < n_kt <= kMappedMaxTiles).
__device__ __forceinline__ void mark(uint32_t* bits, int t0, int t1) {
    if (t0 > t1) return;
    const int w0 = t0 >> 5, w1 = t1 >> 5;
    for (int wd = w0; wd <= w1; ++wd) {
        const int lo = wd == w0 ? (t0 & 31) : 0;
        const int hi = wd == w1 ? (t1 & 31) : 31;
        atomicOr(&bits[wd], (hi == 31 ? 0xffffffffu : ((1u << (hi + 1)) - 1u)) & ~((1u << lo) - 1u));
    }
}

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }   // a >= 0, b >= 1

__global__ __launch_bounds__(kThreads) void mapped_mask_kernel(const MappedParams p) {
    __shared__ uint32_t rbits[kDecisionMaxRowTiles / 32];
    __shared__ uint32_t cbits[kDecisionMaxTiles / 32];
    __shared__ uint32_t tbits[kMappedMaxTiles / 32];
    __shared__ int wave_cnt[kThreads / 64];
    __shared__ int running;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = blockIdx.x % p.n_qt;
    const int map = blockIdx.x / p.n_qt;
    const int d = p.d, T = p.T;
    const int hd = p.h[d], wd_ = p.w[d];
    for (int i = tid; i < kDecisionMaxRowTiles / 32; i += kThreads) rbits[i] = 0;
    for (int i = tid; i < kDecisionMaxTiles / 32; i += kThreads) cbits[i] = 0;
    for (int i = tid; i < kMappedMaxTiles / 32; i += kThreads) tbits[i] = 0;
    if (tid == 0) running = 0;
    __syncthreads();
    // decision row tiles of R's rows
    const int n_t = p.off[T + 1] - p.off[T];
    for (int i = R * kTile + tid; i < min(R * kTile + kTile, n_t); i += kThreads) {
        const int y = i / p.w[T], x = i - y * p.w[T];
        const int dec = (y * hd / p.h[T]) * wd_ + x * wd_ / p.w[T];
        atomicOr(&rbits[(dec / kTile) >> 5], 1u << ((dec / kTile) & 31));
    }
    __syncthreads();
    // kept decision key tiles of any of those row tiles
    const unsigned char* kd = p.kept_d + (int64_t)map * p.n_qt_d * p.n_kt_d;
    for (int c = tid; c < p.n_kt_d; c += kThreads) {
        bool any = false;
        for (int wq = 0; wq < (p.n_qt_d + 31) / 32 && !any; ++wq) {
            uint32_t bitsw = rbits[wq];
            while (bitsw && !any) {
                const int r = wq * 32 + __ffs(bitsw) - 1;
                bitsw &= bitsw - 1u;
                any = kd[(int64_t)r * p.n_kt_d + c] != 0;
            }
        }
        if (any) atomicOr(&cbits[c >> 5], 1u << (c & 31));
    }
    __syncthreads();
    // map every kept decision tile back to the key tiles of step T
    for (int c = tid; c < p.n_kt_d; c += kThreads) {
        if (!((cbits[c >> 5] >> (c & 31)) & 1u)) continue;
        mark(tbits, c, c);                                   // its own tokens (scales <= d)
        const int a = max(c * kTile, p.off[d]) - p.off[d];   // its scale-d tokens [a, e) of grid d
        const int e = min(c * kTile + kTile, p.off[d + 1]) - p.off[d];
        if (a >= e) continue;
        const int y0 = a / wd_, x0 = a - y0 * wd_, y1 = (e - 1) / wd_, x1 = (e - 1) - y1 * wd_;
        // rectangles (ya, yb, xa, xb) of grid d
        int rect[3][4];
        int nrect = 0;
        if (y0 == y1) {
            rect[nrect][0] = y0; rect[nrect][1] = y0; rect[nrect][2] = x0; rect[nrect][3] = x1; ++nrect;
        } else {
            rect[nrect][0] = y0; rect[nrect][1] = y0; rect[nrect][2] = x0; rect[nrect][3] = wd_ - 1; ++nrect;
            if (y1 - y0 > 1) { rect[nrect][0] = y0 + 1; rect[nrect][1] = y1 - 1; rect[nrect][2] = 0; rect[nrect][3] = wd_ - 1; ++nrect; }
            rect[nrect][0] = y1; rect[nrect][1] = y1; rect[nrect][2] = 0; rect[nrect][3] = x1; ++nrect;
        }
        for (int j = d + 1; j <= T; ++j) {
            const int hj = p.h[j], wj = p.w[j];
            for (int q = 0; q < nrect; ++q) {
                const int ylo = cdiv(rect[q][0] * hj, hd), yhi = min(cdiv((rect[q][1] + 1) * hj, hd) - 1, hj - 1);
                const int xlo = cdiv(rect[q][2] * wj, wd_), xhi = min(cdiv((rect[q][3] + 1) * wj, wd_) - 1, wj - 1);
                if (ylo > yhi || xlo > xhi) continue;
                const int base = p.off[j];
                if (xlo == 0 && xhi == wj - 1) {
                    mark(tbits, (base + ylo * wj) / kTile, (base + yhi * wj + wj - 1) / kTile);
                } else {
                    for (int yu = ylo; yu <= yhi; ++yu)
                        mark(tbits, (base + yu * wj + xlo) / kTile, (base + yu * wj + xhi) / kTile);
                }
            }
        }
    }
    __syncthreads();
    // bitmap -> ascending list at col_idx[map][R * n_kt], count at row_ptr[map][R + 1]
    int* out = p.col_idx + (int64_t)map * p.ci_map_stride + (int64_t)R * p.n_kt;
    const int n_words = (p.n_kt + 31) >> 5;
    for (int w0 = 0; w0 < n_words; w0 += kThreads) {
        const int wdx = w0 + tid;
        uint32_t mbits = wdx < n_words ? tbits[wdx] : 0u;
        const int cnt = __popc(mbits);
        int incl = cnt;
#pragma unroll
        for (int dd = 1; dd < 64; dd <<= 1) {
            const int v = __shfl_up(incl, dd);
            if (lane >= dd) incl += v;
        }
        if (lane == 63) wave_cnt[wave] = incl;
        __syncthreads();
        int at = running + incl - cnt;
        for (int w = 0; w < wave; ++w) at += wave_cnt[w];
        while (mbits) {
            out[at++] = wdx * 32 + __ffs(mbits) - 1;
            mbits &= mbits - 1u;
        }
        __syncthreads();
        if (tid == 0) running += wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
        __syncthreads();
    }
    if (tid == 0) {
        int* rp = p.row_ptr + (int64_t)map * p.rp_map_stride;
        rp[R + 1] = running;
        if (R == 0) rp[0] = 0;
    }
}

}  // namespace

hipError_t launch_block_mass(const MassParams& p, int head_dim, hipStream_t s) {
    const int grid = p.B * p.H * p.n_kt;
    if (head_dim == 128) hipLaunchKernelGGL(block_mass_kernel<128>, dim3(grid), dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL(block_mass_kernel<64>, dim3(grid), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_decision(const DecisionParams& p, int rows, hipStream_t s) {
    hipLaunchKernelGGL(decision_kernel, dim3(rows), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_mapped_mask(const MappedParams& p, int maps, hipStream_t s) {
    hipLaunchKernelGGL(mapped_mask_kernel, dim3(maps * p.n_qt), dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    MaskParams c = {};
    c.row_ptr = p.row_ptr;
    c.col_idx = p.col_idx;
    c.n_qt = p.n_qt;
    c.n_kt = p.n_kt;
    c.rp_map_stride = p.rp_map_stride;
    c.ci_map_stride = p.ci_map_stride;
    return launch_mask_compact(c, maps, s);
}

}  // namespace varattn
