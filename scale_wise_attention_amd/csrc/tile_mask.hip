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
// Instead of enumerating pairs, each query row marks the key tiles its
// windows cover.  For key scale j the window is a rectangle of grid j: the
// key rows with y_q*h_j - R_y*h_q <= y_k*h_q <= y_q*h_j + R_y*h_q are
// [ceil((y_q*h_j - R_y*h_q)/h_q), floor((y_q*h_j + R_y*h_q)/h_q)] clipped to
// the grid (same for columns).  Each rectangle row is a run of consecutive
// tokens, so it covers a run of key tiles; a rectangle spanning the full grid
// width is a single run.  The sink scales visible to the row are the token
// prefix [0, off[min(sink_scales, s_q + 1)]).  Window scales below
// sink_scales lie inside that prefix and are skipped.
//
// Two launches: (1) one workgroup per query tile ORs its rows' tile runs into
// a bitmap in LDS and writes the kept columns, in ascending order, at
// col_idx[r*n_kt] with the count in row_ptr[r+1]; (2) one workgroup turns the
// counts into offsets and moves every row's list down to its final place.  A
// mask of at most 2 query tiles takes one launch: one workgroup builds the
// rows in order, each list straight at its final offset.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace varattn {
namespace {

constexpr int kRowThreads = 256;
constexpr int kDirectMaxTiles = 2;     // masks of up to this many query tiles take one launch
constexpr int kChunkTiles = 8192;              // key tiles per bitmap pass
constexpr int kChunkWords = kChunkTiles / 32;

__device__ __forceinline__ int floor_div(int a, int m) { return a >= 0 ? a / m : -((m - 1 - a) / m); }
__device__ __forceinline__ int ceil_div(int a, int m) { return -floor_div(-a, m); }

static_assert(sizeof(MaskBatch) <= 4096, "a mask batch travels as kernel arguments (at most 4 KB)");

// One call of a batch, seen with the field names of MaskParams (the
// schedule arrays point into the batch's kernel arguments).
struct MaskView {
    const int32_t* q_index;
    int32_t n_rows, n_q, q_first, n_kt, num_scales;
    int32_t tile_q, tile_k, sink_scales, local_from_scale, radius_y, radius_x;
    const int32_t* off;
    const int32_t* h;
    const int32_t* w;
};
__device__ __forceinline__ MaskView view_of(const MaskBatch& b, int i) {
    const MaskCall& c = b.c[i];
    return MaskView{c.q_index, c.n_rows, c.n_q, c.q_first, c.n_kt, c.num_scales, b.tile_q, b.tile_k,
                    b.sink_scales, b.local_from_scale, b.radius_y, b.radius_x, b.off, b.h, b.w};
}

// Scale, row and column of query row i of the call (q_index gathered and
// clamped into [0, n_q) so that a bad index cannot read outside the schedule).
template <class P>
__device__ __forceinline__ void row_coords(const P& p, int i, int& s, int& y, int& x) {
    int pos = p.q_index ? p.q_index[i] : i;
    pos = pos < 0 ? 0 : (pos >= p.n_q ? p.n_q - 1 : pos);
    const int tok = p.q_first + pos;
    s = 0;
    while (s + 1 < p.num_scales && tok >= p.off[s + 1]) ++s;
    const int local = tok - p.off[s];
    y = local / p.w[s];
    x = local - y * p.w[s];
}

// Set the bits of key tiles [t0, t1] that fall in the chunk [c0, c0 + kChunkTiles).
__device__ __forceinline__ void mark_tiles(uint32_t* bits, int t0, int t1, int c0) {
    t0 = max(t0 - c0, 0);
    t1 = min(t1 - c0, kChunkTiles - 1);
    if (t0 > t1) return;
    const int w0 = t0 >> 5, w1 = t1 >> 5;
    for (int wd = w0; wd <= w1; ++wd) {
        const int lo = wd == w0 ? (t0 & 31) : 0;
        const int hi = wd == w1 ? (t1 & 31) : 31;
        const uint32_t m = (hi == 31 ? 0xffffffffu : ((1u << (hi + 1)) - 1u)) & ~((1u << lo) - 1u);
        atomicOr(&bits[wd], m);
    }
}

// Scale and grid position of the first kRowThreads rows of a query tile,
// computed once per row (a gathered row costs a load of its index) and read
// by every (row, window scale) item.
struct RowShared {
    uint32_t bits[kChunkWords];
    int wave_cnt[kRowThreads / 64];
    int running;
    int sink_end;
    int rs[kRowThreads], ry[kRowThreads], rx[kRowThreads];
};

// Kept key tiles of query tile r, written in ascending order at out[0 ..);
// returns their count (to every thread).  Keys are processed in chunks of
// kChunkTiles tiles (one pass for every workload up to 8192 key tiles).
template <class P>
__device__ int build_row(const P& p, int r, int* out, RowShared& sh) {
    uint32_t* const bits = sh.bits;
    int* const wave_cnt = sh.wave_cnt;
    int& running = sh.running;
    int& sink_end = sh.sink_end;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i0 = r * p.tile_q;
    const int n_rows = min(p.tile_q, p.n_rows - i0);
    // window scales: [jw, s_q]; scales below sink_scales are covered by the sink prefix
    const int jw = max(p.sink_scales, p.local_from_scale);
    const int nj = max(p.num_scales - jw, 0);
    if (tid == 0) {
        running = 0;
        sink_end = 0;
    }
    // this thread's row (rows past kRowThreads are recomputed where used)
    auto coords = [&](int t, int& s, int& y, int& x) __attribute__((always_inline)) {
        if (t < kRowThreads) {
            s = sh.rs[t];
            y = sh.ry[t];
            x = sh.rx[t];
        } else {
            row_coords(p, i0 + t, s, y, x);
        }
    };
    if (tid < n_rows) row_coords(p, i0 + tid, sh.rs[tid], sh.ry[tid], sh.rx[tid]);
    __syncthreads();
    if (p.sink_scales > 0) {
        int se = 0;
        for (int t = tid; t < n_rows; t += kRowThreads) {
            int s, y, x;
            coords(t, s, y, x);
            se = max(se, p.off[min(p.sink_scales, s + 1)]);
        }
        if (se > 0) atomicMax(&sink_end, se);
    }
    for (int c0 = 0; c0 < p.n_kt; c0 += kChunkTiles) {
        for (int wd = tid; wd < kChunkWords; wd += kRowThreads) bits[wd] = 0;
        __syncthreads();
        if (tid == 0 && sink_end > 0) mark_tiles(bits, 0, (sink_end - 1) / p.tile_k, c0);
        const int n_items = n_rows * nj;
        for (int it = tid; it < n_items; it += kRowThreads) {
            const int t = it / nj;
            const int j = jw + (it - t * nj);
            int s, yq, xq;
            coords(t, s, yq, xq);
            if (j > s) continue;                   // key scale not visible to this row
            const int hq = p.h[s], wq = p.w[s], hj = p.h[j], wj = p.w[j];
            const int ylo = max(ceil_div(yq * hj - p.radius_y * hq, hq), 0);
            const int yhi = min(floor_div(yq * hj + p.radius_y * hq, hq), hj - 1);
            const int xlo = max(ceil_div(xq * wj - p.radius_x * wq, wq), 0);
            const int xhi = min(floor_div(xq * wj + p.radius_x * wq, wq), wj - 1);
            if (ylo > yhi || xlo > xhi) continue;
            const int base = p.off[j];
            if (xlo == 0 && xhi == wj - 1) {
                mark_tiles(bits, (base + ylo * wj) / p.tile_k, (base + yhi * wj + wj - 1) / p.tile_k, c0);
            } else {
                for (int yk = ylo; yk <= yhi; ++yk)
                    mark_tiles(bits, (base + yk * wj + xlo) / p.tile_k, (base + yk * wj + xhi) / p.tile_k, c0);
            }
        }
        __syncthreads();
        // bitmap -> ascending column list (block-wide exclusive scan of popcounts)
        const int n_words = (min(p.n_kt - c0, kChunkTiles) + 31) >> 5;
        for (int w0 = 0; w0 < n_words; w0 += kRowThreads) {
            const int wd = w0 + tid;
            uint32_t m = wd < n_words ? bits[wd] : 0u;
            const int cnt = __popc(m);
            int incl = cnt;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int v = __shfl_up(incl, d);
                if (lane >= d) incl += v;
            }
            if (lane == 63) wave_cnt[wave] = incl;
            __syncthreads();
            int at = running + incl - cnt;
            for (int w = 0; w < wave; ++w) at += wave_cnt[w];
            while (m) {
                const int bit = __ffs(m) - 1;
                out[at++] = c0 + wd * 32 + bit;
                m &= m - 1u;
            }
            __syncthreads();
            if (tid == 0) {
                int tot = 0;
                for (int w = 0; w < kRowThreads / 64; ++w) tot += wave_cnt[w];
                running += tot;
            }
            __syncthreads();
        }
    }
    const int cnt = running;
    __syncthreads();   // every thread has the count before the next row resets it
    return cnt;
}

// One workgroup per query tile; lists at col_idx[r * n_kt], counts in
// row_ptr[r + 1] (moved into place by mask_compact_kernel).
__global__ __launch_bounds__(kRowThreads) void mask_rows_kernel(const MaskParams p) {
    __shared__ RowShared sh;
    const int r = blockIdx.x;
    const int cnt = build_row(p, r, p.col_idx + (int64_t)r * p.n_kt, sh);
    if (threadIdx.x == 0) {
        p.row_ptr[r + 1] = cnt;
        if (r == 0) p.row_ptr[0] = 0;
    }
}

// A mask of few query tiles in one launch: one workgroup builds the rows in
// order and writes each list straight to its final place.
__global__ __launch_bounds__(kRowThreads) void mask_direct_kernel(const MaskParams p) {
    __shared__ RowShared sh;
    int base = 0;
    for (int r = 0; r < p.n_qt; ++r) {
        const int cnt = build_row(p, r, p.col_idx + base, sh);
        base += cnt;
        if (threadIdx.x == 0) p.row_ptr[r + 1] = base;
    }
    if (threadIdx.x == 0) p.row_ptr[0] = 0;
}

// The rows of every call of a batch: workgroup i of the launch builds query
// tile i - first_block[c] of call c (calls without query tiles own no
// workgroup).
__global__ __launch_bounds__(kRowThreads) void mask_rows_batch_kernel(const MaskBatch b) {
    __shared__ RowShared sh;
    int c = 0;
    while (c + 1 < b.n_calls && (int)blockIdx.x >= b.first_block[c + 1]) ++c;
    const MaskView p = view_of(b, c);
    const int r = blockIdx.x - b.first_block[c];
    const int cnt = build_row(p, r, b.c[c].col_idx + (int64_t)r * p.n_kt, sh);
    if (threadIdx.x == 0) {
        b.c[c].row_ptr[r + 1] = cnt;
        if (r == 0) b.c[c].row_ptr[0] = 0;
    }
}

constexpr int kCompactThreads = 1024;
constexpr int kPtrCap = 8192;                  // row offsets staged in LDS up to this many rows
constexpr int kMovePerThread = 4;

// One workgroup per map: counts -> offsets, then move row lists down to their
// final place.  Entry e of the final list (row r, e in [row_ptr[r], row_ptr[r+1]))
// is read from r*n_kt + e - row_ptr[r] >= e.  Entries are moved in chunks:
// all reads of a chunk complete before its writes, and every later chunk
// reads from positions at or beyond its own entries, past what this chunk
// writes, so the in-place move is safe.
struct CompactShared {
    int carry;
    int buf[kCompactThreads];
    int ptr_l[kPtrCap + 1];
    int stage[kCompactThreads * kMovePerThread];
};

// The compaction of one map: n_qt rows of at most n_kt entries at col_idx[r * n_kt].
__device__ void compact_map(int n_qt, int n_kt, int32_t* const row_ptr, int32_t* const col_idx, CompactShared& sh) {
    int& carry = sh.carry;
    int* const buf = sh.buf;
    int* const ptr_l = sh.ptr_l;
    int* const stage = sh.stage;
    const int tid = threadIdx.x;
    const struct {
        int n_qt, n_kt;
    } p{n_qt, n_kt};
    const bool staged = p.n_qt <= kPtrCap;
    if (tid == 0) {
        carry = 0;
        ptr_l[0] = 0;
    }
    __syncthreads();
    // inclusive scan of row_ptr[1..n_qt] in chunks (Hillis-Steele in LDS)
    for (int r0 = 0; r0 < p.n_qt; r0 += kCompactThreads) {
        const int r = r0 + tid;
        buf[tid] = r < p.n_qt ? row_ptr[r + 1] : 0;
        __syncthreads();
        for (int s = 1; s < kCompactThreads; s <<= 1) {
            const int add = tid >= s ? buf[tid - s] : 0;
            __syncthreads();
            buf[tid] += add;
            __syncthreads();
        }
        if (r < p.n_qt) {
            row_ptr[r + 1] = buf[tid] + carry;
            if (staged) ptr_l[r + 1] = buf[tid] + carry;
        }
        __syncthreads();
        if (tid == 0) carry += buf[kCompactThreads - 1];
        __syncthreads();
    }
    if (!staged) {
        // very many query tiles: move row by row
        for (int r = 1; r < p.n_qt; ++r) {
            const int dst = row_ptr[r];
            const int cnt = row_ptr[r + 1] - dst;
            const int64_t src = (int64_t)r * p.n_kt;
            for (int j0 = 0; j0 < cnt; j0 += kCompactThreads) {
                const int j = j0 + tid;
                if (j < cnt) buf[tid] = col_idx[src + j];   // the LDS write waits for the load
                __syncthreads();
                if (j < cnt) col_idx[dst + j] = buf[tid];
                __syncthreads();
            }
        }
        return;
    }
    const int nnz = ptr_l[p.n_qt];
    for (int e0 = 0; e0 < nnz; e0 += kCompactThreads * kMovePerThread) {
        // read the chunk into LDS (a load completes before its LDS write), then write it back
#pragma unroll
        for (int k = 0; k < kMovePerThread; ++k) {
            const int e = e0 + k * kCompactThreads + tid;
            if (e < nnz) {
                // last row r with ptr_l[r] <= e (then e < ptr_l[r + 1])
                int lo = 0, hi = p.n_qt - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (ptr_l[mid] <= e) lo = mid;
                    else hi = mid - 1;
                }
                stage[k * kCompactThreads + tid] = col_idx[(int64_t)lo * p.n_kt + (e - ptr_l[lo])];
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kMovePerThread; ++k) {
            const int e = e0 + k * kCompactThreads + tid;
            if (e < nnz) col_idx[e] = stage[k * kCompactThreads + tid];
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(kCompactThreads) void mask_compact_kernel(const MaskParams p) {
    __shared__ CompactShared sh;
    // one workgroup per map (per (batch, head) for per-head masks)
    compact_map(p.n_qt, p.n_kt, p.row_ptr + (int64_t)blockIdx.x * p.rp_map_stride,
                p.col_idx + (int64_t)blockIdx.x * p.ci_map_stride, sh);
}

// One workgroup per call of a batch; a call without query tiles gets row_ptr = {0}.
__global__ __launch_bounds__(kCompactThreads) void mask_compact_batch_kernel(const MaskBatch b) {
    __shared__ CompactShared sh;
    const MaskCall& c = b.c[blockIdx.x];
    if (c.n_qt == 0) {
        if (threadIdx.x == 0) c.row_ptr[0] = 0;
        return;
    }
    compact_map(c.n_qt, c.n_kt, c.row_ptr, c.col_idx, sh);
}

__global__ void zero_i32_kernel(int32_t* p) { *p = 0; }

}  // namespace

hipError_t launch_zero_i32(int32_t* p, hipStream_t s) {
    hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(1), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_mask_compact(const MaskParams& p, int maps, hipStream_t s) {
    hipLaunchKernelGGL(mask_compact_kernel, dim3(maps), dim3(1024), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_tile_mask_batch(const MaskBatch& b, hipStream_t s) {
    const int blocks = b.first_block[b.n_calls];
    if (blocks > 0) {
        hipLaunchKernelGGL(mask_rows_batch_kernel, dim3(blocks), dim3(kRowThreads), 0, s, b);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(mask_compact_batch_kernel, dim3(b.n_calls), dim3(kCompactThreads), 0, s, b);
    return hipGetLastError();
}

hipError_t launch_tile_mask(const MaskParams& p, hipStream_t s) {
    if (p.n_qt <= kDirectMaxTiles) {
        hipLaunchKernelGGL(mask_direct_kernel, dim3(1), dim3(kRowThreads), 0, s, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(mask_rows_kernel, dim3(p.n_qt), dim3(kRowThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mask_compact_kernel, dim3(1), dim3(1024), 0, s, p);
    return hipGetLastError();
}

}  // namespace varattn
