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
// codes 0x7F / 0xFF are NaN and never produced (x * inv stays within 448 up
// to the rounding of the product, which rounds back to 448).
//
// One workgroup per (tile, map): the tile's pieces (8 bf16 = 16 bytes each)
// stay in registers between the maximum and the encoding, so the tile is
// read from HBM once and its codes written once.  Tiles are independent, so
// a growing key cache requantises only the tiles its new tokens touch.
#include <hip/hip_runtime.h>

#include "e4m3.h"
#include "kernels.h"

namespace varattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTileTokens = 64;
constexpr int kThreads = 256;
constexpr int kMaxPieces = 8;   // pieces per thread: 64 tokens x D/8 pieces over 256 threads, D <= 256

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

    uint32_t w[kMaxPieces][4];
    uint32_t mx = 0u;   // bits of max |x| (non-negative floats order as unsigned integers)
#pragma unroll
    for (int i = 0; i < kMaxPieces; ++i) {
        const int u = threadIdx.x + i * kThreads;
        if (u < pieces) {
            const int r = u / per_row, c = u - r * per_row;
            const u32x4 t = *reinterpret_cast<const u32x4*>(x + (int64_t)(t0 + r) * p.x_st + 8 * c);
            w[i][0] = t.x, w[i][1] = t.y, w[i][2] = t.z, w[i][3] = t.w;
            mx = max(mx, bf16x8_absmax_bits(w[i]));
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
            uint32_t c0, c1;
            bf16x8_to_e4m3(w[i], inv, c0, c1);
            *reinterpret_cast<u32x2*>(out + (int64_t)(t0 + r) * p.c_st + 8 * c) = u32x2{c0, c1};
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
