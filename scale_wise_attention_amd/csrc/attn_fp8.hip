// e4m3 instantiations of the next-scale attention kernel (attn_kernel.h):
// logits from e4m3 queries and keys (the low-bit data precision of "LiteVAR:
// Compressing Visual Autoregressive Modelling with Efficient Attention and
// Quantization"): keys as codes with one scale per 64-token tile, queries
// quantised in the kernel per 64 rows of the call, S^T on the e4m3 matrix
// cores; the weights and v stay bf16, accumulation fp32, fp32 or bf16 output.
#include "attn_kernel.h"

namespace varattn {

int attn_fp8_rows_per_tile(bool sparse) { return sparse ? rows_per_wg<true, 2>() : rows_per_wg<false, 2>(); }

int attn_fp8_resident_wgs(bool out_bf16, bool sparse) {
    if (sparse) return out_bf16 ? resident_wgs<128, true, true, true, 2>() : resident_wgs<128, false, true, true, 2>();
    return out_bf16 ? resident_wgs<128, true, false, true, 2>() : resident_wgs<128, false, false, true, 2>();
}

hipError_t launch_attn_fp8(const AttnParams& p, int D, bool out_bf16, bool sparse, hipStream_t s) {
    if (D != 128) return hipErrorInvalidValue;   // the host layer admits head_dim 128 only
    if (sparse) return out_bf16 ? launch_one<128, true, true, true, 2>(p, s) : launch_one<128, false, true, true, 2>(p, s);
    return out_bf16 ? launch_one<128, true, false, true, 2>(p, s) : launch_one<128, false, false, true, 2>(p, s);
}

}  // namespace varattn
