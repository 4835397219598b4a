// Tile mask (CSR of kept key tiles per query tile) for block-sparse
// next-scale attention.
//
// Rule ("SparVAR: Exploring Sparsity in Visual AutoRegressive Modeling for
// Training-Free Acceleration", abstract: attention sinks, cross-scale
// locality, an index mapping between scales, block-wise sparsity): a pair
// (query of scale q at (y_q, x_q), key of scale j at (y_k, x_k)) with j <= q is
// selected if j < sink_scales, or j >= local_from_scale and
//     |y_q*h_j - y_k*h_q| <= R_y*h_q  and  |x_q*w_j - x_k*w_q| <= R_x*w_q,
// i.e. the key lies within R of the query's position mapped into grid j.
// A tile is kept if it holds one selected pair.
//
// Instead of enumerating pairs, each (query row, key tile) test is closed
// form: the window maps to an integer rectangle [ylo, yhi] x [xlo, xhi] of
// grid j, and the tile's keys of scale j form a row-major interval of that
// grid (a partial first row, full middle rows, a partial last row); the test
// is whether the interval meets the rectangle.
//
// Two launches: (1) one workgroup per query tile tests every key tile, and
// writes its kept columns, compacted in ascending order, at col_idx[r*n_kt]
// with the count in row_ptr[r+1]; (2) one workgroup turns the counts into
// offsets and moves every row's list down to its final place.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace varattn {
namespace {

__device__ __forceinline__ int floor_div(int a, int b) {  // b > 0
    int q = a / b;
    return (a % b != 0 && a < 0) ? q - 1 : q;
}
__device__ __forceinline__ int ceil_div(int a, int b) {   // b > 0
    return -floor_div(-a, b);
}

// Does the row-major interval [p0, p1) of a grid with `w` columns contain a
// point of [ylo, yhi] x [xlo, xhi]?  (p0 < p1; rectangle already clipped.)
__device__ __forceinline__ bool interval_meets_rect(int p0, int p1, int w, int ylo, int yhi, int xlo, int xhi) {
    if (ylo > yhi || xlo > xhi) return false;
    const int y0 = p0 / w, x0 = p0 % w;
    const int y1 = (p1 - 1) / w, x1 = (p1 - 1) % w;
    if (y0 == y1) return y0 >= ylo && y0 <= yhi && max(x0, xlo) <= min(x1, xhi);
    if (y0 >= ylo && y0 <= yhi && max(x0, xlo) <= xhi) return true;          // partial first row
    if (y1 >= ylo && y1 <= yhi && xlo <= min(x1, xhi)) return true;          // partial last row
    return max(y0 + 1, ylo) <= min(y1 - 1, yhi);                              // full middle rows
}

__device__ bool tile_kept(const MaskParams& p, int r, int c) {
    const int k0 = c * p.tile_k;
    const int k1 = min(k0 + p.tile_k, p.kv_len);
    const int i_end = min((r + 1) * p.tile_q, p.n_rows);
    for (int i = r * p.tile_q; i < i_end; ++i) {
        int pos = p.q_index ? p.q_index[i] : i;
        pos = pos < 0 ? 0 : (pos >= p.n_q ? p.n_q - 1 : pos);
        const int t = p.q_first + pos;
        int qs = 0;
        while (qs + 1 < p.num_scales && t >= p.off[qs + 1]) ++qs;
        const int hq = p.h[qs], wq = p.w[qs];
        const int yq = (t - p.off[qs]) / wq, xq = (t - p.off[qs]) % wq;
        // key scales overlapping [k0, k1), visible (j <= qs)
        int j = 0;
        while (j + 1 < p.num_scales && k0 >= p.off[j + 1]) ++j;
        for (; j <= qs && p.off[j] < k1; ++j) {
            const int a = max(k0, p.off[j]) - p.off[j];
            const int e = min(k1, p.off[j + 1]) - p.off[j];
            if (a >= e) continue;
            if (j < p.sink_scales) return true;
            if (j < p.local_from_scale) continue;
            const int hj = p.h[j], wj = p.w[j];
            const int ylo = max(0, ceil_div(yq * hj - p.radius_y * hq, hq));
            const int yhi = min(hj - 1, floor_div(yq * hj + p.radius_y * hq, hq));
            const int xlo = max(0, ceil_div(xq * wj - p.radius_x * wq, wq));
            const int xhi = min(wj - 1, floor_div(xq * wj + p.radius_x * wq, wq));
            if (interval_meets_rect(a, e, wj, ylo, yhi, xlo, xhi)) return true;
        }
    }
    return false;
}

// One workgroup (256 threads) per query tile.
__global__ __launch_bounds__(256) void mask_rows_kernel(const MaskParams p) {
    __shared__ int wave_cnt[4];
    __shared__ int running;
    const int r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) running = 0;
    __syncthreads();
    int* out = p.col_idx + (int64_t)r * p.n_kt;
    for (int c0 = 0; c0 < p.n_kt; c0 += 256) {
        const int c = c0 + tid;
        const bool kept = c < p.n_kt && tile_kept(p, r, c);
        const uint64_t ballot = __ballot(kept);
        const int before = __popcll(ballot & ((1ull << lane) - 1ull));
        if (lane == 0) wave_cnt[wave] = __popcll(ballot);
        __syncthreads();
        int base = running;
        for (int w = 0; w < wave; ++w) base += wave_cnt[w];
        if (kept) out[base + before] = c;
        __syncthreads();
        if (tid == 0) running += wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
        __syncthreads();
    }
    if (tid == 0) {
        p.row_ptr[r + 1] = running;
        if (r == 0) p.row_ptr[0] = 0;
    }
}

// One workgroup: counts -> offsets, then move row lists down in row order.
__global__ __launch_bounds__(1024) void mask_compact_kernel(const MaskParams p) {
    __shared__ int carry;
    const int tid = threadIdx.x;
    // inclusive scan of row_ptr[1..n_qt] in chunks of 1024 (Hillis-Steele in LDS)
    __shared__ int buf[1024];
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int r0 = 0; r0 < p.n_qt; r0 += 1024) {
        const int r = r0 + tid;
        int v = r < p.n_qt ? p.row_ptr[r + 1] : 0;
        buf[tid] = v;
        __syncthreads();
        for (int s = 1; s < 1024; s <<= 1) {
            const int add = tid >= s ? buf[tid - s] : 0;
            __syncthreads();
            buf[tid] += add;
            __syncthreads();
        }
        if (r < p.n_qt) p.row_ptr[r + 1] = buf[tid] + carry;
        __syncthreads();
        if (tid == 0) carry += buf[1023];
        __syncthreads();
    }
    // row_ptr now holds offsets; row r's list sits at r*n_kt, length
    // row_ptr[r+1]-row_ptr[r], and moves down to row_ptr[r] (<= r*n_kt).
    for (int r = 1; r < p.n_qt; ++r) {
        const int dst = p.row_ptr[r];
        const int cnt = p.row_ptr[r + 1] - dst;
        const int64_t src = (int64_t)r * p.n_kt;
        for (int j0 = 0; j0 < cnt; j0 += 1024) {
            const int j = j0 + tid;
            int v = 0;
            if (j < cnt) v = p.col_idx[src + j];
            __syncthreads();
            if (j < cnt) p.col_idx[dst + j] = v;
            __syncthreads();
        }
    }
}

__global__ void zero_i32_kernel(int32_t* p) { *p = 0; }

}  // namespace

hipError_t launch_zero_i32(int32_t* p, hipStream_t s) {
    hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(1), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_tile_mask(const MaskParams& p, hipStream_t s) {
    hipLaunchKernelGGL(mask_rows_kernel, dim3(p.n_qt), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mask_compact_kernel, dim3(1), dim3(1024), 0, s, p);
    return hipGetLastError();
}

}  // namespace varattn
