// bf16 instantiations of the next-scale attention kernel (attn_kernel.h):
// q, k, v in bf16, fp32 accumulation, fp32 or bf16 output.
#include "attn_kernel.h"

namespace varattn {
namespace {
// 32-row query blocks per wave (attn_kernel.h) of the block-sparse head_dim
// 128 kernel (head_dim 64 runs two): one, so two waves share a SIMD.
constexpr int kQBSparse128 = 1;
}  // namespace

int attn_bf16_rows_per_tile(int head_dim, bool sparse, int64_t bh, int64_t rows, int cus) {
    if (sparse) return rows_per_wg<true, 1>();
    if (head_dim == 128) {
        // The 128-row dense workgroup (4 waves of 32 rows, one per SIMD) takes a
        // tile in about 0.7x the time of the 256-row one (4 waves of 64 rows) at
        // half the rows: it wins when its work items all run at once, and loses
        // once they need more rounds of the device than the 256-row items do.
        // Measured on the 1024px steps up to 32x32 (at most 40 key tiles): 7.3 ->
        // 6.4 us (1 tile), 25.0 -> 18.9 us (16x16), 41 -> 36 us (24x24, against 2
        // key splits), 62 -> 58 us (32x32, against 2 splits); 40x40, whose 128-row
        // items take two rounds, stays with 256 rows.
        constexpr int small = rows_per_wg<false, 1>();
        const int64_t items = bh * ((rows + small - 1) / small);
        if (items <= (int64_t)cus * resident_wgs<128, true, false, false, 1>()) return small;
    }
    return rows_per_wg<false, 2>();
}

int attn_bf16_resident_wgs(int D, bool out_bf16, bool sparse, int rows_per_tile) {
    if (sparse) {
        if (D == 128)
            return out_bf16 ? resident_wgs<128, true, true, false, kQBSparse128>()
                            : resident_wgs<128, false, true, false, kQBSparse128>();
        return out_bf16 ? resident_wgs<64, true, true, false, 2>() : resident_wgs<64, false, true, false, 2>();
    }
    if (D == 128 && rows_per_tile == rows_per_wg<false, 1>())
        return out_bf16 ? resident_wgs<128, true, false, false, 1>() : resident_wgs<128, false, false, false, 1>();
    if (D == 128) return out_bf16 ? resident_wgs<128, true, false, false, 2>() : resident_wgs<128, false, false, false, 2>();
    return out_bf16 ? resident_wgs<64, true, false, false, 2>() : resident_wgs<64, false, false, false, 2>();
}

namespace {
// Reconstruction workgroups that follow a block-sparse launch of n_attn
// attention workgroups (cap resident at once): the slots its last round leaves
// free, so that they run beside the attention, at most one per row group.
// With fewer than 64 free slots they would mostly start as the attention
// drains, one group after another, so the attention then runs alone and the
// scatter launch follows it on the stream (the two write disjoint rows).
template <int D, bool OB, int QB, bool WIDE>
hipError_t launch_restore(AttnParams p, int64_t n_attn, int cus, hipStream_t s) {
    constexpr int NT = waves_per_wg<true, QB>() * 64;
    p.rs_rows_per_group = scatter_rows_per_group(p.rs.row_bytes, 16, NT);
    const int64_t n_out = (int64_t)p.rs.h_out * p.rs.w_out;
    const int64_t groups = (int64_t)p.rs.maps * ((n_out + p.rs_rows_per_group - 1) / p.rs_rows_per_group);
    const int64_t cap = (int64_t)cus * resident_wgs<D, OB, true, false, QB, WIDE, true>();
    const int64_t free = n_attn % cap ? cap - n_attn % cap : 0;
    if (free < 64) {
        p.rs_wgs = 0;
        const hipError_t e = launch_one<D, OB, true, false, QB, WIDE>(p, s);
        return e != hipSuccess ? e : launch_scatter(p.rs, s);
    }
    p.rs_wgs = (int)(free < groups ? free : groups);
    return launch_one<D, OB, true, false, QB, WIDE, true>(p, s);
}
}  // namespace

hipError_t launch_attn_bf16(const AttnParams& p, int D, bool out_bf16, bool sparse, int rows_per_tile, int cus,
                            hipStream_t s, bool restore) {
    if (restore) {
        // (block-sparse, unsplit: the reconstruction workgroups follow the attention's)
        if (!sparse || p.n_splits != 1 || rows_per_tile != rows_per_wg<true, 1>()) return hipErrorInvalidValue;
        const int64_t n_attn = (int64_t)p.n_qtiles * p.B * p.H;
        if (D == 128) {
            if (n_attn <= (int64_t)cus * resident_wgs<128, true, true, false, kQBSparse128, true>())
                return out_bf16 ? launch_restore<128, true, kQBSparse128, true>(p, n_attn, cus, s)
                                : launch_restore<128, false, kQBSparse128, true>(p, n_attn, cus, s);
            return out_bf16 ? launch_restore<128, true, kQBSparse128, false>(p, n_attn, cus, s)
                            : launch_restore<128, false, kQBSparse128, false>(p, n_attn, cus, s);
        }
        return out_bf16 ? launch_restore<64, true, 2, false>(p, n_attn, cus, s)
                        : launch_restore<64, false, 2, false>(p, n_attn, cus, s);
    }
    if (sparse) {
        if (rows_per_tile != rows_per_wg<true, 1>()) return hipErrorInvalidValue;
        if (D == 128) {
            // A launch whose workgroups all fit one round at one per compute unit
            // gets the 4-slot ring and tile pairs: its tiles wait on their loads
            // (one tile ahead) more than they share the unit.  Measured on the
            // 1024px sparse steps, one round each, outputs bit-identical: 20x20
            // 28.6 -> 27.0 us, 24x24 36.8 -> 33.5, 32x32 42.7 -> 39.2.
            const int64_t items = (int64_t)p.n_qtiles * p.B * p.H;
            const int64_t grid = p.split_from + (items - p.split_from) * p.n_splits;
            if (grid <= (int64_t)cus * resident_wgs<128, true, true, false, kQBSparse128, true>())
                return out_bf16 ? launch_one<128, true, true, false, kQBSparse128, true>(p, s)
                                : launch_one<128, false, true, false, kQBSparse128, true>(p, s);
            return out_bf16 ? launch_one<128, true, true, false, kQBSparse128>(p, s)
                            : launch_one<128, false, true, false, kQBSparse128>(p, s);
        }
        return out_bf16 ? launch_one<64, true, true, false, 2>(p, s) : launch_one<64, false, true, false, 2>(p, s);
    }
    if (D == 128 && rows_per_tile == rows_per_wg<false, 1>())
        return out_bf16 ? launch_one<128, true, false, false, 1>(p, s) : launch_one<128, false, false, false, 1>(p, s);
    if (rows_per_tile != rows_per_wg<false, 2>()) return hipErrorInvalidValue;
    if (D == 128) return out_bf16 ? launch_one<128, true, false, false, 2>(p, s) : launch_one<128, false, false, false, 2>(p, s);
    return out_bf16 ? launch_one<64, true, false, false, 2>(p, s) : launch_one<64, false, false, false, 2>(p, s);
}

}  // namespace varattn
