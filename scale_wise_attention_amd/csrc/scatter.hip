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
// pointers allow it (else 4 or 2).  The row-group code is in scatter_rows.h.
#include <hip/hip_runtime.h>

#include "kernels.h"
#include "scatter_rows.h"

namespace varattn {
namespace {

constexpr int kThreads = 256;
// Workgroups of a launch at most; each takes every gridDim.x-th group.
constexpr int kMaxBlocks = 8192;

template <int UNIT>
__global__ __launch_bounds__(kThreads) void scatter_kernel(const ScatterParams p, int rows_per_group) {
    scatter_check_index<kThreads>(p, blockIdx.x, gridDim.x);
    __shared__ int src_of[kScatterPasses * kThreads];   // update row of each row of the group, or -1
    scatter_groups<UNIT, kThreads>(p, rows_per_group, blockIdx.x, gridDim.x, src_of);
}

}  // namespace

hipError_t launch_scatter(const ScatterParams& p, hipStream_t s) {
    const int rows_per_group = scatter_rows_per_group(p.row_bytes, p.unit, kThreads);
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
