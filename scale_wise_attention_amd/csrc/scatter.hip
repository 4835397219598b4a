// Structural reconstruction of a pruned grid: out = Scatter(Up(base), I, upd)
// ("ARVAR: Accelerating Visual Autoregressive Model via Attention
// Retrospect", Key Design 3, Equations (8)-(9)).  Up is nearest neighbour
// with source (floor(y*h_in/h_out), floor(x*w_in/w_out)); Scatter overwrites.
//
// One pass over the output grid: every output row picks its single source —
// the update row i if it is retained (marked per group of rows after one
// wave-wide search of the ascending index list), else the upsampled base
// row — so each output byte is written exactly once and no inverse map or
// second pass is needed.  Without update rows (upd NULL) the retained rows
// are skipped: the attention call wrote them in place.  Copies are 16 bytes per lane when rows, strides and
// pointers allow it (else 4 or 2).
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace varattn {
namespace {

constexpr int kThreads = 256;
// Copy passes per row group: a group is as many consecutive rows as 256 lanes
// copy in kPasses passes, so one index search serves kPasses passes of copies.
// (1024px shapes, 128 rows of 256 bytes per group against 16: base-only
// 17.3 -> 13.3 us, full 18.1 -> 14.3 us; 64 rows 13.7 / 14.7, 256 rows 16.2 /
// 18.0, the latter leaving too few workgroups.)
constexpr int kPasses = 8;
// Workgroups of a launch at most; each takes every gridDim.x-th group.
constexpr int kMaxBlocks = 8192;

// First position of the ascending index list holding a value >= t (n if
// none), by one wave: each round probes 64 evenly spaced positions of the
// remaining range [lo, hi] and keeps the gap between the last probe below t
// and the next, so a list of n entries takes about log64(n) rounds of one
// load each (3 for n <= 2^18).  Every round shrinks the range, also for a
// list that is not ascending (the result is then some position in [0, n]).
__device__ __forceinline__ int wave_lower_bound(const int32_t* __restrict__ idx, int n, int t, int lane) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int step = (hi - lo + 63) >> 6;
        const int pos = lo + lane * step;
        const bool below = pos < hi && idx[pos] < t;
        const int c = __popcll(__ballot(below));
        const int nlo = c > 0 ? lo + (c - 1) * step + 1 : lo;
        hi = min(hi, lo + c * step);
        lo = nlo;
    }
    return lo;
}

// A workgroup copies groups of `rows_per_group` consecutive output rows of one
// map (as many rows as 256 lanes cover in kPasses passes, at least one), one
// unit per lane per pass.  Per group, wave 0 finds the group's first retained
// position with one wave-wide search and marks the group's retained rows in LDS.
template <int UNIT>
__global__ __launch_bounds__(kThreads) void scatter_kernel(const ScatterParams p, int rows_per_group) {
    const int n_out = p.h_out * p.w_out;
    const int per_row = p.row_bytes / UNIT;   // the host picks UNIT dividing rows, strides, pointers
    const int groups_per_map = (n_out + rows_per_group - 1) / rows_per_group;
    const int64_t groups = (int64_t)p.maps * groups_per_map;
    const int tid = threadIdx.x;
    // index checks (once, by the first threads of the grid)
    if (p.err_flag) {
        for (int64_t i = (int64_t)blockIdx.x * kThreads + tid; i < p.n_sel; i += (int64_t)gridDim.x * kThreads) {
            const int v = p.q_index[i];
            int bad = 0;
            if (v < 0 || v >= n_out) bad |= 1;
            if (i + 1 < p.n_sel && p.q_index[i + 1] <= v) bad |= 2;
            if (bad) atomicOr(p.err_flag, bad);
        }
    }
    __shared__ int src_of[kPasses * kThreads];   // update row of each row of the group, or -1
    for (int64_t gi = blockIdx.x; gi < groups; gi += gridDim.x) {
        const int m = (int)(gi / groups_per_map);
        const int t0 = (int)(gi - (int64_t)m * groups_per_map) * rows_per_group;
        const int rows = min(rows_per_group, n_out - t0);
        if (tid < 64) {
            for (int r = tid; r < rows; r += 64) src_of[r] = -1;
            if (p.n_sel > 0) {
                // an ascending list holds the group's retained rows in [first, first + rows);
                // with a list that breaks the contract the rows are unspecified but every
                // access stays in bounds
                const int first = wave_lower_bound(p.q_index, p.n_sel, t0, tid);
                for (int r = tid; r < rows; r += 64) {
                    const int k = first + r;
                    if (k < p.n_sel) {
                        const int v = p.q_index[k];
                        if (v >= t0 && v < t0 + rows) src_of[v - t0] = k;
                    }
                }
            }
        }
        __syncthreads();
        const int64_t work = (int64_t)rows * per_row;
        for (int64_t w = tid; w < work; w += kThreads) {
            const int r = (int)(w / per_row);
            const int64_t chunk = w - (int64_t)r * per_row;
            const int t = t0 + r;
            const int i = src_of[r];
            const unsigned char* src;
            if (i >= 0) {
                if (!p.upd) continue;   // a retained row written by the attention call itself
                src = p.upd + m * p.upd_map_stride + (int64_t)i * p.upd_row_stride;
            } else {
                const int y = t / p.w_out, x = t - y * p.w_out;
                const int ys = (int)(((int64_t)y * p.h_in) / p.h_out);
                const int xs = (int)(((int64_t)x * p.w_in) / p.w_out);
                src = p.base + m * p.base_map_stride + (int64_t)(ys * p.w_in + xs) * p.base_row_stride;
            }
            unsigned char* dst = p.out + m * p.out_map_stride + (int64_t)t * p.out_row_stride;
            if constexpr (UNIT == 16) {
                *reinterpret_cast<uint4*>(dst + chunk * 16) = *reinterpret_cast<const uint4*>(src + chunk * 16);
            } else if constexpr (UNIT == 4) {
                *reinterpret_cast<uint32_t*>(dst + chunk * 4) = *reinterpret_cast<const uint32_t*>(src + chunk * 4);
            } else {
                *reinterpret_cast<uint16_t*>(dst + chunk * 2) = *reinterpret_cast<const uint16_t*>(src + chunk * 2);
            }
        }
        __syncthreads();   // the group's marks are read before the next group resets them
    }
}

}  // namespace

hipError_t launch_scatter(const ScatterParams& p, hipStream_t s) {
    const int per_row = p.row_bytes / p.unit;
    const int rows_per_group = per_row >= kPasses * kThreads ? 1 : kPasses * kThreads / per_row;
    const int64_t n_out = (int64_t)p.h_out * p.w_out;
    const int64_t groups = (int64_t)p.maps * ((n_out + rows_per_group - 1) / rows_per_group);
    int64_t blocks = groups < kMaxBlocks ? groups : kMaxBlocks;
    if (blocks < 1) blocks = 1;
    if (p.unit == 16) hipLaunchKernelGGL(scatter_kernel<16>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p, rows_per_group);
    else if (p.unit == 4) hipLaunchKernelGGL(scatter_kernel<4>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p, rows_per_group);
    else hipLaunchKernelGGL(scatter_kernel<2>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p, rows_per_group);
    return hipGetLastError();
}

}  // namespace varattn
