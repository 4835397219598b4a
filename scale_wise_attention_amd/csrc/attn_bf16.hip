// bf16 instantiations of the next-scale attention kernel (attn_kernel.h):
// q, k, v in bf16, fp32 accumulation, fp32 or bf16 output.
#include "attn_kernel.h"

namespace varattn {

int attn_bf16_rows_per_tile(int head_dim, bool sparse) {
    (void)head_dim;
    return (sparse ? waves_per_wg<true>() : waves_per_wg<false>()) * QW;
}

int attn_bf16_resident_wgs(int D, bool out_bf16, bool sparse) {
    if (sparse) {
        if (D == 128) return out_bf16 ? resident_wgs<128, true, true, false>() : resident_wgs<128, false, true, false>();
        return out_bf16 ? resident_wgs<64, true, true, false>() : resident_wgs<64, false, true, false>();
    }
    if (D == 128) return out_bf16 ? resident_wgs<128, true, false, false>() : resident_wgs<128, false, false, false>();
    return out_bf16 ? resident_wgs<64, true, false, false>() : resident_wgs<64, false, false, false>();
}

hipError_t launch_attn_bf16(const AttnParams& p, int D, bool out_bf16, bool sparse, hipStream_t s) {
    if (sparse) {
        if (D == 128) return out_bf16 ? launch_one<128, true, true, false>(p, s) : launch_one<128, false, true, false>(p, s);
        return out_bf16 ? launch_one<64, true, true, false>(p, s) : launch_one<64, false, true, false>(p, s);
    }
    if (D == 128) return out_bf16 ? launch_one<128, true, false, false>(p, s) : launch_one<128, false, false, false>(p, s);
    return out_bf16 ? launch_one<64, true, false, false>(p, s) : launch_one<64, false, false, false>(p, s);
}

}  // namespace varattn
