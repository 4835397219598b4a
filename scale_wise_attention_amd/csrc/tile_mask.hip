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
// form: the tile's keys of scale j form a row-major interval of grid j (a
// partial first row, full middle rows, a partial last row: three
// rectangles), and for a rectangle the window test separates into one test
// per axis: is there a key row y_k in [y0, y1] with y_k*h_q inside
// [y_q*h_j - R*h_q, y_q*h_j + R*h_q] (same for columns)?
//
// Two launches: (1) one workgroup per query tile tests every key tile, and
// writes its kept columns, compacted in ascending order, at col_idx[r*n_kt]
// with the count in row_ptr[r+1]; (2) one workgroup turns the counts into
// offsets and moves every row's list down to its final place.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace varattn {
namespace {

// Is there an integer y in [lo, hi] with a <= y*m <= b  (m >= 1, a <= b)?
// For b - a >= m every long-enough window holds a multiple of m, so the test
// reduces to interval overlap; a shorter window (radius 0) needs the exact check.
__device__ __forceinline__ bool axis_hit(int lo, int hi, int a, int b, int m) {
    if (lo > hi) return false;
    const int L = max(lo * m, a), H = min(hi * m, b);
    if (L > H) return false;
    if (b - a >= m) return true;
    // window shorter than one step: some multiple of m must lie in [L, H]
    const int r = ((L % m) + m) % m;
    return r == 0 || L + (m - r) <= H;
}

// The keys of one scale inside a key tile are the row-major interval from
// (y0, x0) to (y1, x1) of a grid with w columns: up to three rectangles
// (partial first row, full middle rows, partial last row).  Window on key
// rows: ya <= y_k*hq <= yb; on key columns: xa <= x_k*wq <= xb.
__device__ __forceinline__ bool seg_hit(int y0, int x0, int y1, int x1, int w, int ya, int yb, int xa, int xb,
                                        int hq, int wq) {
    if (y0 == y1) return axis_hit(y0, y0, ya, yb, hq) && axis_hit(x0, x1, xa, xb, wq);
    if (axis_hit(y0, y0, ya, yb, hq) && axis_hit(x0, w - 1, xa, xb, wq)) return true;
    if (axis_hit(y1, y1, ya, yb, hq) && axis_hit(0, x1, xa, xb, wq)) return true;
    return axis_hit(y0 + 1, y1 - 1, ya, yb, hq) && axis_hit(0, w - 1, xa, xb, wq);
}

constexpr int kQChunk = 256;   // query rows staged in LDS at a time

// One workgroup (256 threads) per query tile; thread = key tile.  The tile's
// query rows are staged in LDS (scale, y, x) in chunks.  Each thread walks
// the scales present in its key tile, forms that scale's segment once, and
// tests every staged query against it with multiplications and compares.
__global__ __launch_bounds__(256) void mask_rows_kernel(const MaskParams p) {
    __shared__ int wave_cnt[4];
    __shared__ int running;
    __shared__ int qs_l[kQChunk], yq_l[kQChunk], xq_l[kQChunk];
    const int r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) running = 0;
    const int i0 = r * p.tile_q;
    const int i_end = min(i0 + p.tile_q, p.n_rows);
    int* out = p.col_idx + (int64_t)r * p.n_kt;
    for (int c0 = 0; c0 < p.n_kt; c0 += 256) {
        const int c = c0 + tid;
        const bool active = c < p.n_kt;
        const int k0 = c * p.tile_k, k1 = min(k0 + p.tile_k, p.kv_len);
        int j_first = 0;
        if (active)
            while (j_first + 1 < p.num_scales && k0 >= p.off[j_first + 1]) ++j_first;
        bool kept = false;
        for (int q0 = i0; q0 < i_end; q0 += kQChunk) {
            const int nq = min(kQChunk, i_end - q0);
            __syncthreads();
            for (int t = tid; t < nq; t += 256) {
                int pos = p.q_index ? p.q_index[q0 + t] : q0 + t;
                pos = pos < 0 ? 0 : (pos >= p.n_q ? p.n_q - 1 : pos);
                const int tok = p.q_first + pos;
                int qs = 0;
                while (qs + 1 < p.num_scales && tok >= p.off[qs + 1]) ++qs;
                qs_l[t] = qs;
                yq_l[t] = (tok - p.off[qs]) / p.w[qs];
                xq_l[t] = (tok - p.off[qs]) % p.w[qs];
            }
            __syncthreads();
            if (!active || kept) continue;
            for (int j = j_first; j < p.num_scales && p.off[j] < k1 && !kept; ++j) {
                const int a = max(k0, p.off[j]) - p.off[j];
                const int e = min(k1, p.off[j + 1]) - p.off[j];
                if (a >= e) continue;
                const bool sink = j < p.sink_scales;
                if (!sink && j < p.local_from_scale) continue;
                const int hj = p.h[j], wj = p.w[j];
                const int y0 = a / wj, x0 = a % wj, y1 = (e - 1) / wj, x1 = (e - 1) % wj;
                for (int t = 0; t < nq; ++t) {
                    const int qs = qs_l[t];
                    if (j > qs) continue;                 // key scale not visible to this query
                    if (sink) { kept = true; break; }
                    const int hq = p.h[qs], wq = p.w[qs];
                    const int yq = yq_l[t], xq = xq_l[t];
                    const int ya = yq * hj - p.radius_y * hq, yb = yq * hj + p.radius_y * hq;
                    const int xa = xq * wj - p.radius_x * wq, xb = xq * wj + p.radius_x * wq;
                    if (seg_hit(y0, x0, y1, x1, wj, ya, yb, xa, xb, hq, wq)) { kept = true; break; }
                }
            }
        }
        const uint64_t ballot = __ballot(kept && active);
        const int before = __popcll(ballot & ((1ull << lane) - 1ull));
        if (lane == 0) wave_cnt[wave] = __popcll(ballot);
        __syncthreads();
        int base = running;
        for (int w = 0; w < wave; ++w) base += wave_cnt[w];
        if (kept && active) out[base + before] = c;
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
