// e4m3 quantisation of a [B][H][tokens][D] bf16 tensor with one scale per
// (batch, head) map: the low-bit data precision of "LiteVAR: Compressing
// Visual Autoregressive Modelling with Efficient Attention and Quantization"
// (abstract), applied to the attention's queries and keys.
//
//   amax  = max |x| over the map (1 if the map is all zero)
//   code  = e4m3(x * (448 / amax))   fp32 product, round to nearest even,
//                                    magnitudes above 448 saturate to 448
//   scale = amax / 448               dequantised value = e4m3 value * scale
//
// e4m3 is the OCP FP8 "E4M3FN" layout: sign, 4 exponent bits (bias 7),
// 3 mantissa bits, subnormals in multiples of 2^-9, largest finite 448,
// codes 0x7F / 0xFF are NaN and never produced.
//
// Four launches on the caller's stream: clear the per-map maxima (kept as
// float bits in the scale array), the maxima (atomic max of non-negative
// floats as unsigned integers), the codes, and the scales.  HBM-bound: every
// thread moves 16-byte pieces (8 bf16 in, 8 codes out).
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace varattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kUnitsPerThread = 4;   // 8-element pieces per thread and block pass

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> e4m3 code, round to nearest even; |y| above 448 saturates.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t c;
    if (a < 0x3C800000u) {
        // below 2^-6: subnormal codes m * 2^-9 (m = 8 is the smallest normal);
        // the scaling by 2^9 is exact and v_rndne rounds half to even
        c = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    } else {
        // keep 3 of the 23 mantissa bits, round half to even (a carry moves
        // into the exponent), then rebias the exponent from 127 to 7
        c = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
        c = c < 0x7Eu ? c : 0x7Eu;
    }
    return c | sign;
}

__device__ __forceinline__ float map_amax(const QuantParams& p, int m) {
    const float a = __uint_as_float(p.amax_bits[m]);
    return a > 0.f ? a : 1.0f;
}

__global__ __launch_bounds__(kThreads) void quant_clear_kernel(QuantParams p) {
    const int m = blockIdx.x * kThreads + threadIdx.x;
    if (m < p.maps) p.amax_bits[m] = 0u;
}

// piece u of map m: token u / (D/8), elements 8 * (u % (D/8)) .. +7
__device__ __forceinline__ int64_t in_off(const QuantParams& p, int m, int64_t u) {
    const int per_row = p.D / 8;
    const int64_t t = u / per_row;
    const int c = (int)(u - t * per_row);
    const int b = m / p.H, h = m - b * p.H;
    return b * p.x_sb + h * p.x_sh + t * p.x_st + 8 * c;
}
__device__ __forceinline__ int64_t out_off(const QuantParams& p, int m, int64_t u) {
    const int per_row = p.D / 8;
    const int64_t t = u / per_row;
    const int c = (int)(u - t * per_row);
    const int b = m / p.H, h = m - b * p.H;
    return b * p.c_sb + h * p.c_sh + t * p.c_st + 8 * c;
}

__global__ __launch_bounds__(kThreads) void quant_amax_kernel(QuantParams p) {
    const int m = blockIdx.y;
    const int64_t units = (int64_t)p.tokens * (p.D / 8);
    const __bf16* x = reinterpret_cast<const __bf16*>(p.x);
    uint32_t mx = 0u;   // bits of max |x| (non-negative floats order as unsigned integers)
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < units; u += stride) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(x + in_off(p, m, u));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // |bf16| as float bits: clear the sign of both halves
            const uint32_t lo = (w[i] << 16) & 0x7FFFFFFFu;
            const uint32_t hi = w[i] & 0x7FFF0000u;
            mx = max(mx, max(lo, hi));
        }
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, s));
    __shared__ uint32_t red[kThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t v = red[0];
#pragma unroll
        for (int i = 1; i < kThreads / 64; ++i) v = max(v, red[i]);
        if (v) atomicMax(p.amax_bits + m, v);
    }
}

__global__ __launch_bounds__(kThreads) void quant_encode_kernel(QuantParams p) {
    const int m = blockIdx.y;
    const int64_t units = (int64_t)p.tokens * (p.D / 8);
    const float inv = __fdiv_rn(448.0f, map_amax(p, m));
    const __bf16* x = reinterpret_cast<const __bf16*>(p.x);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < units; u += stride) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(x + in_off(p, m, u));
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t c0 = e4m3_code(bf16_lo(w[i]) * inv);
            const uint32_t c1 = e4m3_code(bf16_hi(w[i]) * inv);
            packed[i >> 1] |= (c0 | (c1 << 8)) << (16 * (i & 1));
        }
        *reinterpret_cast<u32x2*>(p.codes + out_off(p, m, u)) = u32x2{packed[0], packed[1]};
    }
}

__global__ __launch_bounds__(kThreads) void quant_scale_kernel(QuantParams p) {
    const int m = blockIdx.x * kThreads + threadIdx.x;
    if (m < p.maps) p.scale[m] = __fdiv_rn(map_amax(p, m), 448.0f);
}

}  // namespace

hipError_t launch_quant_e4m3(const QuantParams& p, hipStream_t s) {
    const unsigned mb = (unsigned)((p.maps + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(quant_clear_kernel, dim3(mb), dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // about 8 blocks per compute unit over all maps, each thread a few pieces
    const int64_t units = (int64_t)p.tokens * (p.D / 8);
    int64_t bx = (units + (int64_t)kThreads * kUnitsPerThread - 1) / ((int64_t)kThreads * kUnitsPerThread);
    const int64_t cap = (2048 + p.maps - 1) / p.maps;
    bx = bx < cap ? bx : cap;
    bx = bx < 1 ? 1 : bx;
    hipLaunchKernelGGL(quant_amax_kernel, dim3((unsigned)bx, (unsigned)p.maps), dim3(kThreads), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(quant_encode_kernel, dim3((unsigned)bx, (unsigned)p.maps), dim3(kThreads), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(quant_scale_kernel, dim3(mb), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace varattn
