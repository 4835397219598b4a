// bf16 instantiations of the next-scale attention kernel (attn_kernel.h):
// q, k, v in bf16, fp32 accumulation, fp32 or bf16 output.
#include "attn_kernel.h"

namespace varattn {
namespace {
// 32-row query blocks per wave (attn_kernel.h): head_dim 128 (dense,
// block-sparse); head_dim 64 always runs two
constexpr int kQBDense128 = 2;
constexpr int kQBSparse128 = 1;
}  // namespace

int attn_bf16_rows_per_tile(int head_dim, bool sparse) {
    (void)head_dim;
    return sparse ? rows_per_wg<true>() : rows_per_wg<false>();
}

int attn_bf16_resident_wgs(int D, bool out_bf16, bool sparse) {
    if (sparse) {
        if (D == 128)
            return out_bf16 ? resident_wgs<128, true, true, false, kQBSparse128>()
                            : resident_wgs<128, false, true, false, kQBSparse128>();
        return out_bf16 ? resident_wgs<64, true, true, false, 2>() : resident_wgs<64, false, true, false, 2>();
    }
    if (D == 128)
        return out_bf16 ? resident_wgs<128, true, false, false, kQBDense128>()
                        : resident_wgs<128, false, false, false, kQBDense128>();
    return out_bf16 ? resident_wgs<64, true, false, false, 2>() : resident_wgs<64, false, false, false, 2>();
}

hipError_t launch_attn_bf16(const AttnParams& p, int D, bool out_bf16, bool sparse, hipStream_t s) {
    if (sparse) {
        if (D == 128)
            return out_bf16 ? launch_one<128, true, true, false, kQBSparse128>(p, s)
                            : launch_one<128, false, true, false, kQBSparse128>(p, s);
        return out_bf16 ? launch_one<64, true, true, false, 2>(p, s) : launch_one<64, false, true, false, 2>(p, s);
    }
    if (D == 128)
        return out_bf16 ? launch_one<128, true, false, false, kQBDense128>(p, s)
                        : launch_one<128, false, false, false, kQBDense128>(p, s);
    return out_bf16 ? launch_one<64, true, false, false, 2>(p, s) : launch_one<64, false, false, false, 2>(p, s);
}

}  // namespace varattn
