// Row copies of the structural reconstruction of a pruned grid ("ARVAR:
// Accelerating Visual Autoregressive Model via Attention Retrospect", Key
// Design 3, Equations (8)-(9)): out = Scatter(Up(base), I, upd), Up nearest
// neighbour with source (floor(y*h_in/h_out), floor(x*w_in/w_out)), Scatter
// overwriting.  Shared by the scatter launch and by the block-sparse
// attention launch that fills the unretained rows in its spare workgroups.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

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
// lane per pass.  Per group, wave 0 writes each row's source into src_of (LDS,
// kScatterPasses * NT ints): -(b + 1) for base row b of the nearest
// upsampling, then, after one wave-wide search of the index list, k >= 0 for a
// row retained as update row k.  Every output row then takes its single
// source: update row k if retained (skipped when upd is NULL: the attention
// call wrote it in place), else the upsampled base row.
template <int UNIT, int NT>
__device__ __forceinline__ void scatter_groups(const ScatterParams& p, int rows_per_group, int64_t wg, int64_t nwg,
                                               int* src_of) {
    const int n_out = p.h_out * p.w_out;
    const int per_row = p.row_bytes / UNIT;   // the host picks UNIT dividing rows, strides, pointers
    const int groups_per_map = (n_out + rows_per_group - 1) / rows_per_group;
    const int64_t groups = (int64_t)p.maps * groups_per_map;
    const int tid = threadIdx.x;
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    typedef typename std::conditional<UNIT == 16, u32x4_t, typename std::conditional<UNIT == 4, uint32_t, uint16_t>::type>::type unit_t;
    for (int64_t gi = wg; gi < groups; gi += nwg) {
        const int m = (int)(gi / groups_per_map);
        const int t0 = (int)(gi - (int64_t)m * groups_per_map) * rows_per_group;
        const int rows = min(rows_per_group, n_out - t0);
        if (tid < 64) {
            for (int r = tid; r < rows; r += 64) {
                const int t = t0 + r;
                const int y = t / p.w_out, x = t - y * p.w_out;
                const int ys = (int)(((int64_t)y * p.h_in) / p.h_out);
                const int xs = (int)(((int64_t)x * p.w_in) / p.w_out);
                src_of[r] = -(ys * p.w_in + xs) - 1;
            }
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
        // kScatterPasses units a lane, all loads issued before the first store
        // (a load-store pair per pass waits one memory round trip each).  The
        // loads are unconditional, from a valid row for every unit (a unit past
        // the group, or of a retained row that is not copied, reads base row 0
        // and stores nothing), so no branch separates them.
        const int work = rows * per_row;   // at most max(kScatterPasses * NT, per_row)
        for (int w0 = tid; w0 < work; w0 += kScatterPasses * NT) {
            unit_t val[kScatterPasses];
            unsigned char* dst[kScatterPasses];
#pragma unroll
            for (int k = 0; k < kScatterPasses; ++k) {
                const int w = w0 + k * NT;
                const bool in = w < work;
                const int r = in ? w / per_row : 0;
                const int chunk = in ? w - r * per_row : 0;
                const int code = in ? src_of[r] : -1;
                const bool from_upd = code >= 0 && p.upd;
                const unsigned char* src =
                    from_upd ? p.upd + m * p.upd_map_stride + (int64_t)code * p.upd_row_stride
                             : p.base + m * p.base_map_stride + (int64_t)(code < 0 ? -code - 1 : 0) * p.base_row_stride;
                val[k] = *reinterpret_cast<const unit_t*>(src + (int64_t)chunk * UNIT);
                // (a retained row without update rows was written by the attention call itself)
                dst[k] = in && (code < 0 || p.upd)
                             ? p.out + m * p.out_map_stride + (int64_t)(t0 + r) * p.out_row_stride + (int64_t)chunk * UNIT
                             : nullptr;
            }
#pragma unroll
            for (int k = 0; k < kScatterPasses; ++k)
                if (dst[k]) *reinterpret_cast<unit_t*>(dst[k]) = val[k];
        }
        __syncthreads();   // the group's marks are read before the next group resets them
    }
}

}  // namespace
}  // namespace varattn
