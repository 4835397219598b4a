// Attention-guided choice of the positions a pruned step recomputes, for gfx950.
//
// "ARVAR: Accelerating Visual Autoregressive Model via Attention Retrospect",
// Key Design 2 and A Worked Example: the attention of an earlier, smaller
// step is reduced to one saliency score per position of its grid, the map is
// interpolated to the grid of the large step and Top-K picks the positions
// to recompute (the retained indices, later gathered by the attention's
// q_index and scattered back by the reconstruction).
//
// Readings where the page is open (it says so itself):
//  * the self-attention part is the block of the step's attention weights
//    (normalised over every key the query sees) whose keys are the step's own
//    tokens, and a position's saliency is the mean of its column over the
//    step's queries;
//  * one map per (batch, head); the selection adds the maps in order in fp32;
//  * nearest interpolation, source floor(dst * in / out) per axis;
//  * larger score first, equal scores by lower position; output ascending.
//
// saliency_kernel: one workgroup per (batch, head, 64 own-scale keys).  The
// logits S^T = K Q^T of the block run on v_mfma_f32_32x32x16_bf16 (keys on M,
// queries on N, as in the attention kernel); each weight is
// exp2(s * scale * log2(e) - lse * log2(e)) with the row's log-sum-exp from
// the attention of the same step, so no second pass over the earlier scales
// is needed.  A lane sums the weights of its queries, the 32 lanes of a
// column block are reduced once at the end, then the 4 waves in order.
//
// select_topk_kernel: one workgroup.  The summed source scores live in LDS as
// order-preserving 32-bit keys; a 4-digit radix select (histogram, then a
// block-wide scan over the digits) finds the key of the n_keep-th best
// position, then one ascending sweep with block-wide scans
// writes the positions above it and the lowest-numbered ones equal to it.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace varattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSalThreads = 256;
constexpr int kSalKeys = 64;     // own-scale keys per workgroup

__device__ __forceinline__ int xcd_spread(int wg, int nwg) {
    // workgroup i runs on XCD i % 8; give each XCD a contiguous range of items
    const int q = nwg >> 3, r = nwg & 7;
    const int x = wg & 7, j = wg >> 3;
    return x * q + (x < r ? x : r) + j;
}

template <int D>
__global__ __launch_bounds__(kSalThreads, 2) void saliency_kernel(const SaliencyParams p) {
    constexpr int SK = D / 16;
    __shared__ float part[kSalThreads / 64][kSalKeys];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, n = lane & 31;
    const int item = xcd_spread(blockIdx.x, gridDim.x);
    const int kb = item % p.n_kb;
    const int bh = item / p.n_kb;
    const int b = bh / p.H, h = bh - b * p.H;

    const __bf16* qbase = reinterpret_cast<const __bf16*>(p.q) + b * p.q_sb + h * p.q_sh;
    const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + b * p.k_sb + h * p.k_sh;
    const float* lse = p.lse + (int64_t)bh * p.n_s;

    // K fragments of the workgroup's 64 keys (A operands, rows clamped to the scale)
    bf16x8 ka[2][SK];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int key = min(kb * kSalKeys + 32 * mb + n, p.n_s - 1);
        const __bf16* kr = kbase + (int64_t)(p.key_first + key) * p.k_st;
#pragma unroll
        for (int ks = 0; ks < SK; ++ks)
            ka[mb][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kr + 16 * ks + 8 * g));
    }
    auto load_q = [&](int qb, bf16x8 (&dst)[SK]) __attribute__((always_inline)) {
        const int row = min(qb * 32 + n, p.n_s - 1);
        const __bf16* qr = qbase + (int64_t)row * p.q_st;
#pragma unroll
        for (int ks = 0; ks < SK; ++ks)
            dst[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qr + 16 * ks + 8 * g));
    };

    float colsum[2][16];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) colsum[mb][r] = 0.f;

    const int n_qb = (p.n_s + 31) / 32;
    constexpr float kLog2e = 1.4426950408889634f;
    bf16x8 qcur[SK], qnext[SK];
    if (wave < n_qb) load_q(wave, qcur);
    for (int qb = wave; qb < n_qb; qb += kSalThreads / 64) {
        const bool more = qb + kSalThreads / 64 < n_qb;
        if (more) load_q(qb + kSalThreads / 64, qnext);
        const int row = qb * 32 + n;
        const bool valid = row < p.n_s;
        // weight = exp2(s * scale*log2e - lse*log2e); rows past the scale get weight 0
        const float shift = valid ? -lse[min(row, p.n_s - 1)] * kLog2e : -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < SK; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[mb][ks], qcur[ks], acc, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) colsum[mb][r] += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[r], p.scale_log2, shift));
        }
        if (more) {
#pragma unroll
            for (int ks = 0; ks < SK; ++ks) qcur[ks] = qnext[ks];
        }
    }
    // sum over the 32 query columns of each half (lanes of equal g)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float v = colsum[mb][r];
#pragma unroll
            for (int m = 1; m < 32; m <<= 1) v += __shfl_xor(v, m);
            colsum[mb][r] = v;
        }
    // lane n of half g stores register r = n & 15 of block mb = n >> 4: key 8(r>>2) + 4g + (r&3)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (n == 16 * mb + r) part[wave][32 * mb + 8 * (r >> 2) + 4 * g + (r & 3)] = colsum[mb][r];
    __syncthreads();
    if (tid < kSalKeys) {
        const int key = kb * kSalKeys + tid;
        if (key < p.n_s) {
            float tot = part[0][tid];
#pragma unroll
            for (int w = 1; w < kSalThreads / 64; ++w) tot += part[w][tid];
            p.sal[(int64_t)bh * p.n_s + key] = tot / (float)p.n_s;
        }
    }
}

constexpr int kSelThreads = 1024;
constexpr int kSelSubHist = 4;

// order-preserving key of a score: larger float -> larger unsigned; -0 counts as +0
__device__ __forceinline__ uint32_t score_key(float f) {
    if (f == 0.f) f = 0.f;
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// block-wide exclusive scan of one int per thread; also returns the block total
__device__ __forceinline__ int block_excl_scan(int v, int* wave_tot, int& total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(incl, d);
        if (lane >= d) incl += t;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
    for (int w = 0; w < kSelThreads / 64; ++w) {
        const int t = wave_tot[w];
        before += w < wave ? t : 0;
        total += t;
    }
    __syncthreads();
    return before + incl - v;
}

__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(const SelectParams p) {
    __shared__ uint32_t src_key[kSelectMaxSrc];
    __shared__ uint32_t dst_key[kSelectDstCache];
    __shared__ int hist[256 * kSelSubHist];
    __shared__ int wave_tot[kSelThreads / 64];
    __shared__ uint32_t sh_prefix;
    __shared__ int sh_need;
    const int tid = threadIdx.x;
    const int n_src = p.h_src * p.w_src;
    const int n_dst = p.h_dst * p.w_dst;
    const bool cached = n_dst <= kSelectDstCache;
    // summed source scores, maps added in order (loads issued 8 at a time)
    for (int s = tid; s < n_src; s += kSelThreads) {
        float acc = 0.f;
        for (int m0 = 0; m0 < p.maps; m0 += 8) {
            float t[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) t[i] = m0 + i < p.maps ? p.sal[(int64_t)(m0 + i) * n_src + s] : 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (m0 + i < p.maps) acc += t[i];
        }
        src_key[s] = score_key(acc);
    }
    __syncthreads();
    // nearest source of destination t (all products below 2^24)
    auto src_of = [&](int t) __attribute__((always_inline)) -> int {
        const int y = t / p.w_dst, x = t - y * p.w_dst;
        return (y * p.h_src / p.h_dst) * p.w_src + x * p.w_src / p.w_dst;
    };
    if (cached)
        for (int t = tid; t < n_dst; t += kSelThreads) dst_key[t] = src_key[src_of(t)];
    auto key_of = [&](int t) __attribute__((always_inline)) -> uint32_t {
        return cached ? dst_key[t] : src_key[src_of(t)];
    };
    if (tid == 0) {
        sh_prefix = 0u;
        sh_need = p.n_keep;
    }
    __syncthreads();
    // radix select of the n_keep-th largest key, 8 bits at a time from the top;
    // 4 sub-histograms (by wave) spread the LDS atomics
    uint32_t mask = 0u;
    const int sub = (tid >> 6) & (kSelSubHist - 1);
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256 * kSelSubHist; i += kSelThreads) hist[i] = 0;
        __syncthreads();
        const uint32_t prefix = sh_prefix;
        const int need = sh_need;
        for (int t = tid; t < n_dst; t += kSelThreads) {
            const uint32_t k = key_of(t);
            if ((k & mask) == prefix) atomicAdd(&hist[sub * 256 + ((k >> shift) & 255u)], 1);
        }
        __syncthreads();
        // thread i < 256 holds digit 255 - i; an exclusive scan in that order gives,
        // per digit, the count of keys with a larger digit
        int cnt = 0;
        if (tid < 256)
            for (int j = 0; j < kSelSubHist; ++j) cnt += hist[j * 256 + 255 - tid];
        int total;
        const int larger = block_excl_scan(cnt, wave_tot, total);
        if (tid < 256 && larger < need && larger + cnt >= need) {
            sh_need = need - larger;              // still to take among keys with this digit
            sh_prefix = prefix | ((uint32_t)(255 - tid) << shift);
        }
        mask |= 255u << shift;
        __syncthreads();
    }
    const uint32_t thr = sh_prefix;   // key of the n_keep-th best position
    const int take_eq = sh_need;      // positions with key == thr to keep, lowest first
    // ascending sweep: keep key > thr, and the first take_eq positions with key == thr
    int eq_before = 0, out_at = 0;
    for (int t0 = 0; t0 < n_dst; t0 += kSelThreads) {
        const int t = t0 + tid;
        const uint32_t k = t < n_dst ? key_of(t) : 0u;
        const bool eq = t < n_dst && k == thr;
        int eq_tot;
        const int eq_rank = eq_before + block_excl_scan(eq ? 1 : 0, wave_tot, eq_tot);
        const bool keep = t < n_dst && (k > thr || (eq && eq_rank < take_eq));
        int kept_tot;
        const int at = out_at + block_excl_scan(keep ? 1 : 0, wave_tot, kept_tot);
        if (keep && at < p.n_keep) p.q_index[at] = t;   // at < n_keep by construction
        eq_before += eq_tot;
        out_at += kept_tot;
    }
}

}  // namespace

hipError_t launch_saliency(const SaliencyParams& p, int head_dim, hipStream_t s) {
    const int grid = p.B * p.H * p.n_kb;
    if (head_dim == 128) hipLaunchKernelGGL(saliency_kernel<128>, dim3(grid), dim3(kSalThreads), 0, s, p);
    else hipLaunchKernelGGL(saliency_kernel<64>, dim3(grid), dim3(kSalThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_select_topk(const SelectParams& p, hipStream_t s) {
    hipLaunchKernelGGL(select_topk_kernel, dim3(1), dim3(kSelThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace varattn
