// Block-causal next-scale attention with float32 inputs (small head dims).
//
// Same definition as the bf16 kernels (each query sees all keys of its own
// and earlier scales, "SparVAR: Exploring Sparsity in Visual AutoRegressive
// Modeling for Training-Free Acceleration", abstract), computed in fp32 on the
// vector ALUs: one wave per 64 query rows, one lane per query, K/V staged in
// LDS 32 keys at a time and read as broadcasts.  This path exists for fp32
// callers and small problems; the throughput path is the bf16 MFMA kernel.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace varattn {
namespace {

constexpr int KH = 32;   // keys per LDS stage (half of a 64-key tile)

template <int D, bool SPARSE>
__global__ __launch_bounds__(64) void attn_f32_kernel(const AttnParams p) {
    __shared__ __attribute__((aligned(16))) float Ks[KH][D];
    __shared__ __attribute__((aligned(16))) float Vs[KH][D];
    const int lane = threadIdx.x;
    const int qtile = blockIdx.x % p.n_qtiles;
    const int bh = blockIdx.x / p.n_qtiles;
    const int b = bh / p.H, h = bh - b * p.H;

    const int my_row = qtile * 64 + lane;
    const bool row_valid = my_row < p.n_rows;
    const int row_c = row_valid ? my_row : p.n_rows - 1;
    int pos = p.q_index ? p.q_index[row_c] : row_c;
    pos = pos < 0 ? 0 : (pos >= p.n_q ? p.n_q - 1 : pos);
    const int tok = p.q_first + pos;
    int klim = p.kv_len;
    if (!p.step_mode) {
#pragma unroll
        for (int s = VAR_MAX_SCALES - 1; s >= 0; --s)
            if (s < p.num_scales && tok < p.scale_end[s]) klim = p.scale_end[s];
    }
    int wmax = klim;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) wmax = max(wmax, __shfl_xor(wmax, m));

    const float* qp = reinterpret_cast<const float*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)pos * p.q_st;
    float qv[D], o[D];
#pragma unroll
    for (int d = 0; d < D; d += 4) {
        const float4 t = *reinterpret_cast<const float4*>(qp + d);
        qv[d] = t.x; qv[d + 1] = t.y; qv[d + 2] = t.z; qv[d + 3] = t.w;
        o[d] = o[d + 1] = o[d + 2] = o[d + 3] = 0.f;
    }
    const float* kp = reinterpret_cast<const float*>(p.k) + b * p.k_sb + h * p.k_sh;
    const float* vp = reinterpret_cast<const float*>(p.v) + b * p.v_sb + h * p.v_sh;
    const float c2 = p.scale_log2;
    float m = -INFINITY, l = 0.f;   // m in log2 units

    int n_tiles, list_begin = 0;
    if constexpr (SPARSE) {
        list_begin = p.row_ptr[qtile];
        n_tiles = p.row_ptr[qtile + 1] - list_begin;
    } else {
        n_tiles = (wmax + 63) / 64;
    }
    for (int it = 0; it < n_tiles; ++it) {
        // (a column repeated right after itself is visited once; the list is uniform)
        if (SPARSE && it > 0 && p.col_idx[list_begin + it] == p.col_idx[list_begin + it - 1]) continue;
        const int tbase = SPARSE ? min(max(p.col_idx[list_begin + it], 0), (p.kv_len - 1) / 64) * 64 : it * 64;
        for (int half = 0; half < 2; ++half) {
            const int kbase = tbase + half * KH;
            __syncthreads();
            for (int e = lane * 4; e < KH * D; e += 64 * 4) {
                const int r = e / D, d = e % D;
                const int key = min(kbase + r, p.kv_len - 1);
                *reinterpret_cast<float4*>(&Ks[r][d]) = *reinterpret_cast<const float4*>(kp + (int64_t)key * p.k_st + d);
                *reinterpret_cast<float4*>(&Vs[r][d]) = *reinterpret_cast<const float4*>(vp + (int64_t)key * p.v_st + d);
            }
            __syncthreads();
            for (int j = 0; j < KH; ++j) {
                const int key = kbase + j;
                if (key >= klim) break;
                float s = 0.f;
#pragma unroll
                for (int d = 0; d < D; ++d) s = __builtin_fmaf(qv[d], Ks[j][d], s);
                s *= c2;
                if (s > m) {
                    const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - s);
#pragma unroll
                    for (int d = 0; d < D; ++d) o[d] *= alpha;
                    l *= alpha;
                    m = s;
                }
                const float pr = exp2f(s - m);
                l += pr;
#pragma unroll
                for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(pr, Vs[j][d], o[d]);
            }
        }
    }
    if (row_valid) {
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        float* op = reinterpret_cast<float*>(p.o) + b * p.o_sb + h * p.o_sh + (int64_t)out_row_of(p, my_row) * p.o_st;
#pragma unroll
        for (int d = 0; d < D; d += 4)
            *reinterpret_cast<float4*>(op + d) = make_float4(o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv);
        if (p.lse)
            p.lse[(int64_t)(b * p.H + h) * p.n_rows + my_row] = l > 0.f ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
    }
}

template <int D, bool SP>
hipError_t launch_one(const AttnParams& p, hipStream_t s) {
    hipLaunchKernelGGL((attn_f32_kernel<D, SP>), dim3(p.n_qtiles * p.B * p.H), dim3(64), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const AttnParams& p, int D, bool sparse, hipStream_t s) {
    if (D == 32) return sparse ? launch_one<32, true>(p, s) : launch_one<32, false>(p, s);
    return sparse ? launch_one<64, true>(p, s) : launch_one<64, false>(p, s);
}

}  // namespace varattn
