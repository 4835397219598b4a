// bf16 instantiations of the next-scale attention kernel (attn_kernel.h):
// q, k, v in bf16, fp32 accumulation, fp32 or bf16 output.
#include "attn_kernel.h"

namespace varattn {
namespace {
// 32-row query blocks per wave (attn_kernel.h) of the head_dim 128 kernels;
// head_dim 64 always runs two.  Block-sparse: one.  Dense: one for launches
// whose workgroups walk at most kShortWalk key tiles, two otherwise.  One
// block per wave (two waves per SIMD) shortens a tile's latency; over a long
// launch its extra LDS reads and instructions cost more clock (the chip is
// then power-limited) than the overlap gains.  Measured on the 1024px steps:
// steps up to 32x32 (at most 20 tiles per workgroup after key splits) 4-13%
// faster with one block, 40x40 and larger (65+ tiles) 2-3% slower.
constexpr int kQBSparse128 = 1;
constexpr int kShortWalk = 32;

int dense_qb128(const AttnParams& p) {
    const int n_kt = (p.kv_len + KT - 1) / KT;
    const int items = p.n_qtiles * p.B * p.H;
    // tiles of the longest walk: a whole item's, unless every item is split
    const int walk = (p.split_from == 0 && items > 0) ? (n_kt + p.n_splits - 1) / p.n_splits : n_kt;
    return walk <= kShortWalk ? 1 : 2;
}
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
    // (one workgroup per compute unit with either block count: the 4-slot ring)
    if (D == 128) return out_bf16 ? resident_wgs<128, true, false, false, 2>() : resident_wgs<128, false, false, false, 2>();
    return out_bf16 ? resident_wgs<64, true, false, false, 2>() : resident_wgs<64, false, false, false, 2>();
}

hipError_t launch_attn_bf16(const AttnParams& p, int D, bool out_bf16, bool sparse, hipStream_t s) {
    if (sparse) {
        if (D == 128)
            return out_bf16 ? launch_one<128, true, true, false, kQBSparse128>(p, s)
                            : launch_one<128, false, true, false, kQBSparse128>(p, s);
        return out_bf16 ? launch_one<64, true, true, false, 2>(p, s) : launch_one<64, false, true, false, 2>(p, s);
    }
    if (D == 128) {
        if (dense_qb128(p) == 1)
            return out_bf16 ? launch_one<128, true, false, false, 1>(p, s) : launch_one<128, false, false, false, 1>(p, s);
        return out_bf16 ? launch_one<128, true, false, false, 2>(p, s) : launch_one<128, false, false, false, 2>(p, s);
    }
    return out_bf16 ? launch_one<64, true, false, false, 2>(p, s) : launch_one<64, false, false, false, 2>(p, s);
}

}  // namespace varattn
