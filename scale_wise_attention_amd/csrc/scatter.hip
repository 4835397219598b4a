// Structural reconstruction of a pruned grid: out = Scatter(Up(base), I, upd)
// ("ARVAR: Accelerating Visual Autoregressive Model via Attention
// Retrospect", Key Design 3, Equations (8)-(9)).  Up is nearest neighbour
// with source (floor(y*h_in/h_out), floor(x*w_in/w_out)); Scatter overwrites.
//
// One pass over the output grid: every output row picks its single source —
// the update row i if it is retained (found by binary search in the
// ascending index list), else the upsampled base row — so each output byte is
// written exactly once and no inverse map or second pass is needed.  Copies
// are 16 bytes per lane when rows, strides and pointers allow it (else 4 or 2).
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace varattn {
namespace {

// Index of t in the ascending list, or -1.
__device__ __forceinline__ int find_index(const int32_t* __restrict__ idx, int n, int t) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (idx[mid] < t) lo = mid + 1; else hi = mid;
    }
    return (lo < n && idx[lo] == t) ? lo : -1;
}

template <int UNIT>
__global__ __launch_bounds__(256) void scatter_kernel(const ScatterParams p) {
    const int n_out = p.h_out * p.w_out;
    const int per_row = p.row_bytes / UNIT;   // the host picks UNIT dividing rows, strides, pointers
    const int64_t total = (int64_t)p.maps * n_out * per_row;
    // index checks (once, by the first threads of the grid)
    if (p.err_flag) {
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < p.n_sel;
             i += (int64_t)gridDim.x * blockDim.x) {
            const int v = p.q_index[i];
            int bad = 0;
            if (v < 0 || v >= n_out) bad |= 1;
            if (i + 1 < p.n_sel && p.q_index[i + 1] <= v) bad |= 2;
            if (bad) atomicOr(p.err_flag, bad);
        }
    }
    for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < total;
         it += (int64_t)gridDim.x * blockDim.x) {
        const int chunk = (int)(it % per_row);
        const int64_t rowlin = it / per_row;
        const int t = (int)(rowlin % n_out);
        const int m = (int)(rowlin / n_out);
        const int i = find_index(p.q_index, p.n_sel, t);
        const unsigned char* src;
        if (i >= 0) {
            src = p.upd + m * p.upd_map_stride + i * p.upd_row_stride;
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
}

}  // namespace

hipError_t launch_scatter(const ScatterParams& p, hipStream_t s) {
    const int64_t total = (int64_t)p.maps * p.h_out * p.w_out * (p.row_bytes / p.unit);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    if (p.unit == 16) hipLaunchKernelGGL(scatter_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, s, p);
    else if (p.unit == 4) hipLaunchKernelGGL(scatter_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(scatter_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace varattn
