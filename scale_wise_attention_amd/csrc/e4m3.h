// bf16 -> OCP e4m3 ("E4M3FN": sign, 4 exponent bits with bias 7, 3 mantissa
// bits, subnormals in multiples of 2^-9, largest finite 448, no infinities)
// for values already scaled into [-448, 448] (up to the rounding of the
// scaling product): round to nearest even, with subnormals, by
// v_cvt_pk_fp8_f32 (two values per instruction).  Shared by the quantiser
// and the attention kernel that quantises its queries.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace varattn {

// Largest magnitude of the 8 bf16 values in w, as float bits (non-negative
// floats order as unsigned integers).
__device__ __forceinline__ uint32_t bf16x8_absmax_bits(const uint32_t (&w)[4]) {
    uint32_t m = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t lo = (w[j] << 16) & 0x7FFFFFFFu, hi = w[j] & 0x7FFF0000u;
        m = max(m, max(lo, hi));
    }
    return m;
}

// e4m3 codes of the 8 bf16 values in w times inv (fp32 products), packed 4
// per dword in order; |w| * inv must not exceed 448 beyond rounding.
__device__ __forceinline__ void bf16x8_to_e4m3(const uint32_t (&w)[4], float inv, uint32_t& out0, uint32_t& out1) {
    int packed[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t a = w[2 * j], b = w[2 * j + 1];
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(a << 16) * inv, __uint_as_float(a & 0xFFFF0000u) * inv,
                                                0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(b << 16) * inv, __uint_as_float(b & 0xFFFF0000u) * inv, v,
                                            true);
        packed[j] = v;
    }
    out0 = (uint32_t)packed[0];
    out1 = (uint32_t)packed[1];
}

}  // namespace varattn
