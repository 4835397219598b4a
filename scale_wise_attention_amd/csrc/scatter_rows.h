// Row copies of the structural reconstruction of a pruned grid ("ARVAR:
// Accelerating Visual Autoregressive Model via Attention Retrospect", Key
// Design 3, Equations (8)-(9)): out = Scatter(Up(base), I, upd), Up nearest
// neighbour with source (floor(y*h_in/h_out), floor(x*w_in/w_out)), Scatter
// overwriting.  Shared by the scatter launch and by the block-sparse
// attention launch that fills the unretained rows in its spare workgroups.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace varattn {
namespace {

// Copy passes per row group: a group is as many consecutive rows as a
// workgroup's lanes copy in kScatterPasses passes, so one index search serves
// that many passes of copies.  (1024px shapes, 128 rows of 256 bytes per
// group against 16: base-only 17.3 -> 13.3 us, full 18.1 -> 14.3 us; 64 rows
// 13.7 / 14.7, 256 rows 16.2 / 18.0, the latter leaving too few workgroups.)
constexpr int kScatterPasses = 8;

// Rows per group for rows of row_bytes bytes copied `unit` bytes a lane by
// `threads` lanes.
__host__ __device__ inline int scatter_rows_per_group(int row_bytes, int unit, int threads) {
    const int per_row = row_bytes / unit;
    return per_row >= kScatterPasses * threads ? 1 : kScatterPasses * threads / per_row;
}

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

// Index checks: workgroup `wg` of `nwg` looks at its share of the list and
// ORs 1 (out of range) or 2 (not strictly ascending) into err_flag.
template <int NT>
__device__ __forceinline__ void scatter_check_index(const ScatterParams& p, int64_t wg, int64_t nwg) {
    if (!p.err_flag) return;
    const int n_out = p.h_out * p.w_out;
    for (int64_t i = wg * NT + threadIdx.x; i < p.n_sel; i += nwg * NT) {
        const int v = p.q_index[i];
        int bad = 0;
        if (v < 0 || v >= n_out) bad |= 1;
        if (i + 1 < p.n_sel && p.q_index[i + 1] <= v) bad |= 2;
        if (bad) atomicOr(p.err_flag, bad);
    }
}

// Workgroup `wg` of `nwg` (NT lanes) copies every nwg-th group of
// `rows_per_group` consecutive output rows of one map, one UNIT-byte unit per
// lane per pass.  Per group, wave 0 finds the group's first retained position
// with one wave-wide search and marks the group's retained rows in src_of
// (LDS, kScatterPasses * NT ints); every output row then takes its single
// source: update row i if retained (skipped when upd is NULL: the attention
// call wrote it in place), else the upsampled base row.
template <int UNIT, int NT>
__device__ __forceinline__ void scatter_groups(const ScatterParams& p, int rows_per_group, int64_t wg, int64_t nwg,
                                               int* src_of) {
    const int n_out = p.h_out * p.w_out;
    const int per_row = p.row_bytes / UNIT;   // the host picks UNIT dividing rows, strides, pointers
    const int groups_per_map = (n_out + rows_per_group - 1) / rows_per_group;
    const int64_t groups = (int64_t)p.maps * groups_per_map;
    const int tid = threadIdx.x;
    for (int64_t gi = wg; gi < groups; gi += nwg) {
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
        for (int64_t w = tid; w < work; w += NT) {
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
}  // namespace varattn
