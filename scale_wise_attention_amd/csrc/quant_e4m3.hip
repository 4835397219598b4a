// e4m3 quantisation of a [B][H][tokens][D] bf16 tensor with one scale per
// (batch, head, 64-token tile): the low-bit data precision of "LiteVAR:
// Compressing Visual Autoregressive Modelling with Efficient Attention and
// Quantization" (abstract), applied to the attention's queries and keys.
// For each tile (its <= 64 tokens x D values):
//
//   amax  = max |x| over the tile (1 if the tile is all zero)
//   code  = e4m3(x * (448 / amax))   fp32 product, round to nearest even,
//                                    magnitudes above 448 saturate to 448
//   scale = amax / 448               dequantised value = e4m3 value * scale
//
// e4m3 is the OCP FP8 "E4M3FN" layout: sign, 4 exponent bits (bias 7),
// 3 mantissa bits, subnormals in multiples of 2^-9, largest finite 448,
// codes 0x7F / 0xFF are NaN and never produced.
//
// One workgroup per (tile, map): the tile's pieces (8 bf16 = 16 bytes each)
// stay in registers between the maximum and the encoding, so the tile is
// read from HBM once and its codes written once.  Tiles are independent, so
// a growing key cache requantises only the tiles its new tokens touch.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace varattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTileTokens = 64;
constexpr int kThreads = 256;
constexpr int kMaxPieces = 8;   // pieces per thread: 64 tokens x D/8 pieces over 256 threads, D <= 256

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

__global__ __launch_bounds__(kThreads) void quant_tile_kernel(const QuantParams p) {
    const int m = blockIdx.y;
    const int tile = p.tile_first + blockIdx.x;
    const int b = m / p.H, h = m - b * p.H;
    const int per_row = p.D / 8;
    const int t0 = tile * kTileTokens;
    const int rows = min(kTileTokens, p.tokens - t0);
    const int pieces = rows * per_row;
    const __bf16* x = reinterpret_cast<const __bf16*>(p.x) + b * p.x_sb + h * p.x_sh;
    uint8_t* out = p.codes + b * p.c_sb + h * p.c_sh;

    u32x4 w[kMaxPieces];
    uint32_t mx = 0u;   // bits of max |x| (non-negative floats order as unsigned integers)
#pragma unroll
    for (int i = 0; i < kMaxPieces; ++i) {
        const int u = threadIdx.x + i * kThreads;
        w[i] = u32x4{0u, 0u, 0u, 0u};
        if (u < pieces) {
            const int r = u / per_row, c = u - r * per_row;
            w[i] = *reinterpret_cast<const u32x4*>(x + (int64_t)(t0 + r) * p.x_st + 8 * c);
#pragma unroll
            for (int j = 0; j < 4; ++j) mx = max(mx, max((w[i][j] << 16) & 0x7FFFFFFFu, w[i][j] & 0x7FFF0000u));
        }
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, s));
    __shared__ uint32_t red[kThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) mx = max(mx, red[i]);
    const float amax = mx ? __uint_as_float(mx) : 1.0f;
    const float inv = __fdiv_rn(448.0f, amax);
#pragma unroll
    for (int i = 0; i < kMaxPieces; ++i) {
        const int u = threadIdx.x + i * kThreads;
        if (u < pieces) {
            const int r = u / per_row, c = u - r * per_row;
            uint32_t packed[2] = {0u, 0u};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t c0 = e4m3_code(bf16_lo(w[i][j]) * inv);
                const uint32_t c1 = e4m3_code(bf16_hi(w[i][j]) * inv);
                packed[j >> 1] |= (c0 | (c1 << 8)) << (16 * (j & 1));
            }
            *reinterpret_cast<u32x2*>(out + (int64_t)(t0 + r) * p.c_st + 8 * c) = u32x2{packed[0], packed[1]};
        }
    }
    if (threadIdx.x == 0) p.scale[m * p.scale_stride + tile] = __fdiv_rn(amax, 448.0f);
}

}  // namespace

hipError_t launch_quant_e4m3(const QuantParams& p, hipStream_t s) {
    const int n_tiles = (p.tokens + kTileTokens - 1) / kTileTokens - p.tile_first;
    if (n_tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(quant_tile_kernel, dim3((unsigned)n_tiles, (unsigned)p.maps), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace varattn
