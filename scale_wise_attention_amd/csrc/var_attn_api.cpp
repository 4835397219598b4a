// C-ABI host layer of libvarattn.so (declared in include/var_attn.h).
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime, derives the schedule offsets, fills the kernel's parameter
// block and enqueues the kernel(s) on the caller's stream.  Nothing is
// allocated, nothing is cached between calls.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kernels.h"

#define VAR_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[512] = "";

var_status fail(var_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

var_status ok() {
    g_last_error[0] = '\0';
    return VAR_OK;
}

var_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(VAR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

struct Offsets {
    int32_t off[VAR_MAX_SCALES + 1];
    int32_t num_scales;
};

constexpr int64_t kMaxTokens = 1 << 24;

var_status check_schedule(const var_schedule* s, Offsets* o) {
    if (!s) return fail(VAR_ERR_NULL, "schedule is NULL");
    if (s->num_scales < 1 || s->num_scales > VAR_MAX_SCALES)
        return fail(VAR_ERR_SCHEDULE, "num_scales=%d outside [1, %d]", s->num_scales, VAR_MAX_SCALES);
    if (!s->h || !s->w) return fail(VAR_ERR_NULL, "schedule h or w is NULL");
    int64_t acc = 0;
    o->off[0] = 0;
    for (int k = 0; k < s->num_scales; ++k) {
        if (s->h[k] < 1 || s->h[k] > 4096 || s->w[k] < 1 || s->w[k] > 4096)
            return fail(VAR_ERR_SCHEDULE, "scale %d has grid %dx%d outside [1, 4096]", k, s->h[k], s->w[k]);
        acc += (int64_t)s->h[k] * s->w[k];
        if (acc >= kMaxTokens) return fail(VAR_ERR_SCHEDULE, "schedule exceeds %lld tokens", (long long)kMaxTokens);
        o->off[k + 1] = (int32_t)acc;
    }
    o->num_scales = s->num_scales;
    return VAR_OK;
}

var_status check_range(const Offsets& o, int32_t b, int32_t e) {
    if (b < 0 || e > o.num_scales || b >= e)
        return fail(VAR_ERR_RANGE, "scale range [%d, %d) invalid for %d scales", b, e, o.num_scales);
    return VAR_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

var_status check_layout(const char* name, const var_layout& l, int D, int elem_bytes) {
    const int64_t m = 16 / elem_bytes;   // elements per 16 bytes
    if (l.batch < 0 || l.head < 0 || l.token < D)
        return fail(VAR_ERR_STRIDE, "%s strides (%lld, %lld, %lld) invalid for head_dim %d", name,
                    (long long)l.batch, (long long)l.head, (long long)l.token, D);
    if (l.batch % m || l.head % m || l.token % m)
        return fail(VAR_ERR_STRIDE, "%s strides must be multiples of %lld elements", name, (long long)m);
    // the kernels address the rows of one 64-key tile with 32-bit byte offsets
    if (l.token * elem_bytes * 64 >= ((int64_t)1 << 31))
        return fail(VAR_ERR_STRIDE, "%s token stride %lld too large", name, (long long)l.token);
    return VAR_OK;
}

// Common validation + parameter fill for the two attention entry points.
var_status prepare_attn(const var_schedule* sched, const var_attn_desc* d, const void* q, var_layout ql,
                        const void* k, var_layout kl, const void* v, var_layout vl, void* o, var_layout ol,
                        float* lse, const int32_t* q_index, int32_t n_sel, varattn::AttnParams* p,
                        bool* nothing_to_do) {
    *nothing_to_do = false;
    Offsets off;
    var_status st = check_schedule(sched, &off);
    if (st != VAR_OK) return st;
    if (!d) return fail(VAR_ERR_NULL, "desc is NULL");
    st = check_range(off, d->q_scale_begin, d->q_scale_end);
    if (st != VAR_OK) return st;
    if (d->batch < 1 || d->heads < 1 || (int64_t)d->batch * d->heads > (1 << 20))
        return fail(VAR_ERR_RANGE, "batch=%d heads=%d invalid", d->batch, d->heads);
    if (d->in_dtype == VAR_BF16) {
        if (d->head_dim != 64 && d->head_dim != 128)
            return fail(VAR_ERR_UNSUPPORTED, "bf16 input supports head_dim 64 or 128, got %d", d->head_dim);
        if (d->out_dtype != VAR_F32 && d->out_dtype != VAR_BF16)
            return fail(VAR_ERR_UNSUPPORTED, "unknown out_dtype %d", (int)d->out_dtype);
    } else if (d->in_dtype == VAR_F32) {
        if (d->head_dim != 32 && d->head_dim != 64)
            return fail(VAR_ERR_UNSUPPORTED, "f32 input supports head_dim 32 or 64, got %d", d->head_dim);
        if (d->out_dtype != VAR_F32)
            return fail(VAR_ERR_UNSUPPORTED, "f32 input requires f32 output");
    } else {
        return fail(VAR_ERR_UNSUPPORTED, "unknown in_dtype %d", (int)d->in_dtype);
    }
    if (!(d->softmax_scale >= 0.f) || std::isinf(d->softmax_scale))
        return fail(VAR_ERR_RANGE, "softmax_scale must be finite and >= 0 (0 = 1/sqrt(D))");
    const int32_t first = off.off[d->q_scale_begin];
    const int32_t n_q = off.off[d->q_scale_end] - first;
    int32_t rows = n_q;
    if (q_index) {
        if (n_sel < 0 || n_sel > n_q) return fail(VAR_ERR_INDEX, "n_sel=%d outside [0, n_q=%d]", n_sel, n_q);
        rows = n_sel;
    } else if (n_sel != 0) {
        return fail(VAR_ERR_INDEX, "n_sel=%d given without q_index", n_sel);
    }
    if (d->out_at_index != 0 && d->out_at_index != 1)
        return fail(VAR_ERR_RANGE, "out_at_index must be 0 or 1");
    if (d->out_at_index && !q_index) return fail(VAR_ERR_INDEX, "out_at_index needs q_index");
    if (rows == 0) {   // nothing to compute; o and lse may be empty (NULL) tensors
        *nothing_to_do = true;
        return ok();
    }
    if (!q || !k || !v || !o) return fail(VAR_ERR_NULL, "q, k, v and o must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(VAR_ERR_STRIDE, "q, k, v and o must be 16-byte aligned");
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(VAR_ERR_STRIDE, "lse must be 4-byte aligned");
    const int ib = d->in_dtype == VAR_BF16 ? 2 : 4;
    const int ob = d->out_dtype == VAR_BF16 ? 2 : 4;
    if ((st = check_layout("q", ql, d->head_dim, ib)) != VAR_OK) return st;
    if ((st = check_layout("k", kl, d->head_dim, ib)) != VAR_OK) return st;
    if ((st = check_layout("v", vl, d->head_dim, ib)) != VAR_OK) return st;
    // the bf16 output is written 4 elements (8 bytes) at a time, f32 4 at a time (16 bytes)
    if (ol.batch < 0 || ol.head < 0 || ol.token < d->head_dim || ol.batch % 4 || ol.head % 4 || ol.token % 4)
        return fail(VAR_ERR_STRIDE, "o strides must be non-negative multiples of 4 elements, token >= head_dim");
    (void)ob;
    std::memset(p, 0, sizeof(*p));
    p->q = q; p->k = k; p->v = v; p->o = o; p->lse = lse; p->q_index = q_index;
    p->q_sb = ql.batch; p->q_sh = ql.head; p->q_st = ql.token;
    p->k_sb = kl.batch; p->k_sh = kl.head; p->k_st = kl.token;
    p->v_sb = vl.batch; p->v_sh = vl.head; p->v_st = vl.token;
    p->o_sb = ol.batch; p->o_sh = ol.head; p->o_st = ol.token;
    p->B = d->batch; p->H = d->heads;
    p->n_rows = rows; p->n_q = n_q; p->q_first = first;
    p->kv_len = off.off[d->q_scale_end];
    p->num_scales = d->q_scale_end;   // scales beyond the call's last are never visible
    p->step_mode = (d->q_scale_end - d->q_scale_begin == 1) ? 1 : 0;
    p->out_at_index = d->out_at_index;
    const float scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / std::sqrt((float)d->head_dim);
    p->scale = scale;
    p->scale_log2 = scale * 1.4426950408889634f;
    for (int s = 0; s < VAR_MAX_SCALES; ++s) p->scale_end[s] = s < off.num_scales ? off.off[s + 1] : off.off[off.num_scales];
    p->n_splits = 1;
    return ok();
}

// Split items and partial rows of a launch with `items` work items of `rpt`
// rows (bh maps of `rows` rows each) on `cap` resident workgroups: the items
// that fill whole rounds run unsplit (split_from = items / cap * cap); the
// partial rows are those of the split items, numbered in the flattened
// (map, row) order from the first row of item split_from on.
struct SplitRows {
    int64_t split_from, part_first, part_rows;
};
SplitRows split_rows(int64_t bh, int64_t rows, int64_t rpt, int64_t cap) {
    const int64_t n_qt = (rows + rpt - 1) / rpt, items = bh * n_qt;
    SplitRows r;
    r.split_from = items / cap * cap;
    r.part_first = r.split_from >= items ? bh * rows : (r.split_from / n_qt) * rows + (r.split_from % n_qt) * rpt;
    r.part_rows = bh * rows - r.part_first;
    return r;
}

// Bytes of the split workspace the kernels use: fp32 O and LSE per split and
// partial row.
int64_t split_need_bytes(int32_t splits, int64_t part_rows, int32_t D) {
    return splits > 1 ? (int64_t)splits * part_rows * (D + 1) * 4 : 0;
}

// Records a split request after its basic checks; the workspace size is
// checked by set_split_items once the split items are known.
var_status attach_splits(varattn::AttnParams* p, const var_attn_desc* d, int32_t splits, void* ws) {
    if (splits < 1 || splits > varattn::kMaxSplits)
        return fail(VAR_ERR_RANGE, "n_splits=%d outside [1, %d]", splits, varattn::kMaxSplits);
    if (splits == 1) return VAR_OK;
    if (d->in_dtype != VAR_BF16) return fail(VAR_ERR_UNSUPPORTED, "key splits need bf16 input");
    if (!ws) return fail(VAR_ERR_NULL, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(ws) & 15u) return fail(VAR_ERR_STRIDE, "workspace must be 16-byte aligned");
    p->n_splits = splits;
    p->part_o = static_cast<float*>(ws);
    return VAR_OK;
}

// Compute units and peak engine clock (kHz) of the current device, read once
// per device.  From the device properties record (its layout is versioned in
// the HIP ABI), not from hipDeviceGetAttribute, whose attribute numbers differ
// between HIP runtime releases (the process may run on another release of the
// runtime than these headers describe).  {0, 0} when there is no device.
struct DeviceInfo {
    int cus, clock_khz;
};
DeviceInfo device_info() {
    constexpr int kMaxDevices = 64;
    static std::atomic<long long> cache[kMaxDevices];   // cus << 32 | clock_khz, 0 = not read yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return {0, 0};
    }
    if (dev < kMaxDevices) {
        const long long c = cache[dev].load(std::memory_order_relaxed);
        if (c) return {(int)(c >> 32), (int)(c & 0xffffffff)};
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return {0, 0};
    }
    const DeviceInfo r{prop.multiProcessorCount, prop.clockRate};
    if (dev < kMaxDevices && r.cus > 0)
        cache[dev].store(((long long)r.cus << 32) | (unsigned)r.clock_khz, std::memory_order_relaxed);
    return r;
}

int device_cu_count() {
    const int n = device_info().cus;
    return n > 0 ? n : 256;
}

// Items of a key-split launch: those that fill whole rounds of the device's
// resident workgroups run unsplit (split_from); only the remaining partial
// round is split (every item when there are fewer than one round's worth).
// Checks that the launch grid stays below 2^31 and that the workspace holds
// the split items' partial rows, and points part_o / part_lse into it.
var_status set_split_items(varattn::AttnParams* p, int resident_per_cu, int rpt, int D, int64_t ws_bytes) {
    const int64_t items = (int64_t)p->n_qtiles * p->B * p->H;
    int64_t from = items;
    if (p->n_splits > 1) {
        const SplitRows r = split_rows((int64_t)p->B * p->H, p->n_rows, rpt,
                                       (int64_t)device_cu_count() * resident_per_cu);
        from = r.split_from;
        const int64_t need = split_need_bytes(p->n_splits, r.part_rows, D);
        if (ws_bytes < need)
            return fail(VAR_ERR_CAPACITY, "workspace of %lld bytes below the %lld needed", (long long)ws_bytes,
                        (long long)need);
        p->part_first = r.part_first;
        p->part_rows = r.part_rows;
        p->part_lse = p->part_o + p->n_splits * r.part_rows * D;
    }
    if (from + (items - from) * p->n_splits >= ((int64_t)1 << 31)) return fail(VAR_ERR_RANGE, "launch grid too large");
    p->split_from = (int32_t)from;
    return VAR_OK;
}

// Split count: the fewest splits whose modelled time is within 3% of the
// lowest (the model's noise).  Time is counted in units of one 64-key
// iteration of a workgroup (about 1.8 us on MI355X at the 1024px shapes).
// The items that fill whole rounds of the `cap` resident workgroups run
// unsplit, a round taking `tiles` iterations; the rest, split s ways, take
// their rounds of ceil(tiles / s) iterations, plus the merge: a launch (about
// 3 iterations) and the split items' partial O written and read back (8 bytes
// per element; about 7 MB per iteration at the bandwidth these small launches
// reach).
int32_t choose_splits(int64_t tasks, int64_t tiles, int64_t bh_rows, int32_t D, int64_t cap) {
    auto rounds = [&](int64_t n) { return (n + cap - 1) / cap; };
    const int64_t whole = tasks / cap * cap, rest = tasks - whole;
    if (rest == 0) return 1;
    const double rest_rows = (double)bh_rows * rest / tasks;
    double cost[varattn::kMaxSplits + 1];
    cost[1] = (double)rounds(tasks) * tiles;
    double lowest = cost[1];
    int32_t s_max = 1;
    for (int32_t s = 2; s <= varattn::kMaxSplits && tiles >= 2 * s; ++s) {
        cost[s] = (double)(whole / cap) * tiles + (double)rounds(rest * s) * ((tiles + s - 1) / s) + 3.0 +
                  (double)s * rest_rows * D * 8.0 / 7.2e6;
        lowest = cost[s] < lowest ? cost[s] : lowest;
        s_max = s;
    }
    // the fewest splits within 3% of the lowest modelled cost (the model's noise)
    for (int32_t s = 1; s <= s_max; ++s)
        if (cost[s] <= 1.03 * lowest) return s;
    return 1;
}

}  // namespace

VAR_EXPORT const char* var_status_string(var_status s) {
    switch (s) {
        case VAR_OK: return "VAR_OK";
        case VAR_ERR_NULL: return "VAR_ERR_NULL";
        case VAR_ERR_SCHEDULE: return "VAR_ERR_SCHEDULE";
        case VAR_ERR_RANGE: return "VAR_ERR_RANGE";
        case VAR_ERR_UNSUPPORTED: return "VAR_ERR_UNSUPPORTED";
        case VAR_ERR_STRIDE: return "VAR_ERR_STRIDE";
        case VAR_ERR_CAPACITY: return "VAR_ERR_CAPACITY";
        case VAR_ERR_INDEX: return "VAR_ERR_INDEX";
        case VAR_ERR_HIP: return "VAR_ERR_HIP";
    }
    return "VAR_ERR_UNKNOWN";
}

VAR_EXPORT const char* var_last_error(void) { return g_last_error; }

VAR_EXPORT var_status var_device_info(int32_t* compute_units, int32_t* max_clock_khz) {
    const DeviceInfo d = device_info();
    if (d.cus <= 0) return fail(VAR_ERR_HIP, "no current HIP device");
    if (compute_units) *compute_units = d.cus;
    if (max_clock_khz) *max_clock_khz = d.clock_khz;
    return ok();
}

VAR_EXPORT var_status var_schedule_extent(const var_schedule* sched, int32_t b, int32_t e, int64_t* first_token,
                                          int64_t* n_q, int64_t* kv_len) {
    Offsets off;
    var_status st = check_schedule(sched, &off);
    if (st != VAR_OK) return st;
    if ((st = check_range(off, b, e)) != VAR_OK) return st;
    if (first_token) *first_token = off.off[b];
    if (n_q) *n_q = off.off[e] - off.off[b];
    if (kv_len) *kv_len = off.off[e];
    return ok();
}

namespace {

// Tile scales of e4m3 keys: k_scale[m][k_stride] covers the call's
// ceil(kv_len / 64) key tiles.
struct E4m3Keys {
    const float* scale;
    int64_t stride;
};

// Extra checks of a call whose k is e4m3 codes (q and v bf16): head_dim 128,
// 16-byte strides of the code tensor, a scale array present and long enough.
// p is the filled parameter block (kv_len known).
var_status check_e4m3(const var_attn_desc* desc, var_layout k_l, const E4m3Keys& kc,
                      const varattn::AttnParams& p) {
    if (desc->in_dtype != VAR_BF16 || desc->head_dim != 128)
        return fail(VAR_ERR_UNSUPPORTED, "e4m3 keys need bf16 q and v (in_dtype) and head_dim 128");
    if (!kc.scale) return fail(VAR_ERR_NULL, "k_scale must be non-NULL");
    if (reinterpret_cast<uintptr_t>(kc.scale) & 3u) return fail(VAR_ERR_STRIDE, "k_scale must be 4-byte aligned");
    if (kc.stride < (p.kv_len + 63) / 64)
        return fail(VAR_ERR_STRIDE, "k_scale_stride=%lld below the %d key tiles of the call", (long long)kc.stride,
                    (p.kv_len + 63) / 64);
    return check_layout("k", k_l, desc->head_dim, 1);
}

void attach_e4m3(varattn::AttnParams* p, const E4m3Keys& kc) {
    p->k_scale = kc.scale;
    p->k_scale_stride = kc.stride;
}

var_status dense_impl(const var_schedule* sched, const var_attn_desc* desc, const void* q, var_layout q_l,
                      const void* k, var_layout k_l, const void* v, var_layout v_l, void* o, var_layout o_l,
                      float* lse, const int32_t* q_index, int32_t n_sel, int32_t splits, void* ws,
                      int64_t ws_bytes, void* stream, const E4m3Keys* e4m3 = nullptr) {
    varattn::AttnParams p;
    bool none = false;
    var_status st = prepare_attn(sched, desc, q, q_l, k, k_l, v, v_l, o, o_l, lse, q_index, n_sel, &p, &none);
    if (st != VAR_OK) return st;
    if (e4m3 && !none && (st = check_e4m3(desc, k_l, *e4m3, p)) != VAR_OK) return st;
    if ((st = attach_splits(&p, desc, none ? 1 : splits, ws)) != VAR_OK) return st;
    if (none) return ok();
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (e4m3) {
        attach_e4m3(&p, *e4m3);
        const int rpt = varattn::attn_fp8_rows_per_tile(false);
        p.n_qtiles = (p.n_rows + rpt - 1) / rpt;
        if ((st = set_split_items(&p, varattn::attn_fp8_resident_wgs(desc->out_dtype == VAR_BF16, false), rpt,
                                  desc->head_dim, ws_bytes)) != VAR_OK)
            return st;
        return hip_status(varattn::launch_attn_fp8(p, desc->head_dim, desc->out_dtype == VAR_BF16, false, s),
                          "var_attn_dense_e4m3 launch");
    }
    if (desc->in_dtype == VAR_BF16) {
        const int rpt = varattn::attn_bf16_rows_per_tile(desc->head_dim, false, (int64_t)p.B * p.H, p.n_rows,
                                                         device_cu_count());
        p.n_qtiles = (p.n_rows + rpt - 1) / rpt;
        const bool ob = desc->out_dtype == VAR_BF16;
        if ((st = set_split_items(&p, varattn::attn_bf16_resident_wgs(desc->head_dim, ob, false, rpt), rpt,
                                  desc->head_dim, ws_bytes)) != VAR_OK)
            return st;
        return hip_status(varattn::launch_attn_bf16(p, desc->head_dim, ob, false, rpt, device_cu_count(), s),
                          "var_attn_dense launch");
    }
    p.n_qtiles = (p.n_rows + varattn::kF32RowsPerTile - 1) / varattn::kF32RowsPerTile;
    return hip_status(varattn::launch_attn_f32(p, desc->head_dim, false, s), "var_attn_dense launch");
}

var_status sparse_impl(const var_schedule* sched, const var_attn_desc* desc, const void* q, var_layout q_l,
                       const void* k, var_layout k_l, const void* v, var_layout v_l, void* o, var_layout o_l,
                       float* lse, const int32_t* q_index, int32_t n_sel, const int32_t* row_ptr,
                       const int32_t* col_idx, int32_t tile_q, int32_t tile_k, int32_t splits, void* ws,
                       int64_t ws_bytes, void* stream, int64_t col_bh_stride = -1,
                       const E4m3Keys* e4m3 = nullptr, const varattn::ScatterParams* restore = nullptr) {
    if (tile_q != 64 || tile_k != 64)
        return fail(VAR_ERR_UNSUPPORTED, "block-sparse attention supports 64x64 tiles, got %dx%d", tile_q, tile_k);
    if (!row_ptr || !col_idx) return fail(VAR_ERR_NULL, "row_ptr and col_idx must be non-NULL");
    varattn::AttnParams p;
    bool none = false;
    var_status st = prepare_attn(sched, desc, q, q_l, k, k_l, v, v_l, o, o_l, lse, q_index, n_sel, &p, &none);
    if (st != VAR_OK) return st;
    if (e4m3 && !none && (st = check_e4m3(desc, k_l, *e4m3, p)) != VAR_OK) return st;
    if ((st = attach_splits(&p, desc, none ? 1 : splits, ws)) != VAR_OK) return st;
    if (none) return ok();
    p.row_ptr = row_ptr;
    p.col_idx = col_idx;
    if (col_bh_stride >= 0) {   // one CSR per (batch, head)
        if (desc->in_dtype != VAR_BF16) return fail(VAR_ERR_UNSUPPORTED, "per-head CSR needs bf16 v");
        const int64_t n_qt = (p.n_rows + 63) / 64;
        const int64_t n_kt = (p.kv_len + 63) / 64;
        if (col_bh_stride < n_qt * n_kt)
            return fail(VAR_ERR_CAPACITY, "col_stride=%lld below n_qt*n_kt=%lld", (long long)col_bh_stride,
                        (long long)(n_qt * n_kt));
        p.rp_bh_stride = n_qt + 1;
        p.ci_bh_stride = col_bh_stride;
    }
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (desc->in_dtype == VAR_BF16) {
        // each workgroup covers a whole number of 64-row tiles of the mask
        const int rpt = e4m3 ? varattn::attn_fp8_rows_per_tile(true)
                             : varattn::attn_bf16_rows_per_tile(desc->head_dim, true, (int64_t)p.B * p.H, p.n_rows,
                                                                device_cu_count());
        p.n_qtiles = (p.n_rows + rpt - 1) / rpt;
        const bool ob = desc->out_dtype == VAR_BF16;
        const int resident = e4m3 ? varattn::attn_fp8_resident_wgs(ob, true)
                                  : varattn::attn_bf16_resident_wgs(desc->head_dim, ob, true, rpt);
        if ((st = set_split_items(&p, resident, rpt, desc->head_dim, ws_bytes)) != VAR_OK) return st;
        if (e4m3) {
            attach_e4m3(&p, *e4m3);
            return hip_status(varattn::launch_attn_fp8(p, desc->head_dim, desc->out_dtype == VAR_BF16, true, s),
                              "var_attn_block_sparse_e4m3 launch");
        }
        if (restore) {
            p.rs = *restore;
            return hip_status(varattn::launch_attn_bf16(p, desc->head_dim, ob, true, rpt, device_cu_count(), s, true),
                              "var_attn_block_sparse_restore launch");
        }
        return hip_status(varattn::launch_attn_bf16(p, desc->head_dim, ob, true, rpt, device_cu_count(), s),
                          "var_attn_block_sparse launch");
    }
    p.n_qtiles = (p.n_rows + varattn::kF32RowsPerTile - 1) / varattn::kF32RowsPerTile;
    return hip_status(varattn::launch_attn_f32(p, desc->head_dim, true, s), "var_attn_block_sparse launch");
}

}  // namespace

VAR_EXPORT var_status var_attn_dense(const var_schedule* sched, const var_attn_desc* desc, const void* q,
                                     var_layout q_l, const void* k, var_layout k_l, const void* v, var_layout v_l,
                                     void* o, var_layout o_l, float* lse, const int32_t* q_index, int32_t n_sel,
                                     void* stream) {
    return dense_impl(sched, desc, q, q_l, k, k_l, v, v_l, o, o_l, lse, q_index, n_sel, 1, nullptr, 0, stream);
}

VAR_EXPORT var_status var_attn_block_sparse(const var_schedule* sched, const var_attn_desc* desc, const void* q,
                                            var_layout q_l, const void* k, var_layout k_l, const void* v,
                                            var_layout v_l, void* o, var_layout o_l, float* lse,
                                            const int32_t* q_index, int32_t n_sel, const int32_t* row_ptr,
                                            const int32_t* col_idx, int32_t tile_q, int32_t tile_k,
                                            void* stream) {
    return sparse_impl(sched, desc, q, q_l, k, k_l, v, v_l, o, o_l, lse, q_index, n_sel, row_ptr, col_idx, tile_q,
                       tile_k, 1, nullptr, 0, stream);
}

VAR_EXPORT var_status var_attn_block_sparse_restore(const var_schedule* sched, const var_attn_desc* desc,
                                                    const void* q, var_layout q_l, const void* k, var_layout k_l,
                                                    const void* v, var_layout v_l, void* o, var_layout o_l,
                                                    float* lse, const int32_t* q_index, int32_t n_sel,
                                                    const int32_t* row_ptr, const int32_t* col_idx, int32_t tile_q,
                                                    int32_t tile_k, const void* base, var_layout base_l,
                                                    int32_t h_in, int32_t w_in, int32_t* err_flag, void* stream) {
    Offsets off;
    var_status st = check_schedule(sched, &off);
    if (st != VAR_OK) return st;
    if (!desc) return fail(VAR_ERR_NULL, "desc is NULL");
    if ((st = check_range(off, desc->q_scale_begin, desc->q_scale_end)) != VAR_OK) return st;
    if (desc->q_scale_end != desc->q_scale_begin + 1)
        return fail(VAR_ERR_RANGE, "the reconstruction covers one step: q_scale_end must be q_scale_begin + 1");
    if (desc->in_dtype != VAR_BF16) return fail(VAR_ERR_UNSUPPORTED, "the reconstruction call takes bf16 input");
    if (desc->out_at_index != 1) return fail(VAR_ERR_RANGE, "the reconstruction call needs out_at_index = 1");
    if (desc->out_dtype != VAR_F32 && desc->out_dtype != VAR_BF16)
        return fail(VAR_ERR_UNSUPPORTED, "unknown out_dtype %d", (int)desc->out_dtype);
    if (desc->head_dim != 64 && desc->head_dim != 128)
        return fail(VAR_ERR_UNSUPPORTED, "bf16 input supports head_dim 64 or 128, got %d", desc->head_dim);
    if (desc->batch < 1 || desc->heads < 1 || (int64_t)desc->batch * desc->heads > (1 << 20))
        return fail(VAR_ERR_RANGE, "batch=%d heads=%d invalid", desc->batch, desc->heads);
    if (h_in < 1 || w_in < 1 || (int64_t)h_in * w_in >= kMaxTokens) return fail(VAR_ERR_RANGE, "base grid invalid");
    if (!base || !o) return fail(VAR_ERR_NULL, "base and o must be non-NULL");
    const int eb = desc->out_dtype == VAR_BF16 ? 2 : 4;
    const int D = desc->head_dim;
    // rows are copied 16 bytes a lane: every row start must be 16-byte aligned
    const int64_t bs[3] = {base_l.batch, base_l.head, base_l.token}, os[3] = {o_l.batch, o_l.head, o_l.token};
    for (int i = 0; i < 3; ++i)
        if (bs[i] < 0 || os[i] < 0 || (bs[i] * eb) % 16 || (os[i] * eb) % 16)
            return fail(VAR_ERR_STRIDE, "o and base strides must be non-negative multiples of 16 bytes");
    if (!aligned16(base) || !aligned16(o)) return fail(VAR_ERR_STRIDE, "o and base must be 16-byte aligned");
    if (base_l.token < D || o_l.token < D) return fail(VAR_ERR_STRIDE, "token strides must be >= head_dim");
    // map m = b * heads + h at m * head stride: batch stride = heads * head stride (any when batch = 1)
    if (desc->batch > 1 && (o_l.batch != (int64_t)desc->heads * o_l.head || base_l.batch != (int64_t)desc->heads * base_l.head))
        return fail(VAR_ERR_STRIDE, "o and base need batch stride = heads * head stride");
    varattn::ScatterParams r;
    std::memset(&r, 0, sizeof(r));
    r.base = static_cast<const unsigned char*>(base);
    r.upd = nullptr;
    r.out = static_cast<unsigned char*>(o);
    r.q_index = q_index;
    r.err_flag = err_flag;
    r.base_map_stride = base_l.head * eb;
    r.base_row_stride = base_l.token * eb;
    r.out_map_stride = o_l.head * eb;
    r.out_row_stride = o_l.token * eb;
    r.maps = desc->batch * desc->heads;
    r.row_bytes = D * eb;
    r.n_sel = n_sel;
    r.h_in = h_in;
    r.w_in = w_in;
    r.h_out = sched->h[desc->q_scale_begin];
    r.w_out = sched->w[desc->q_scale_begin];
    r.unit = 16;
    if (n_sel < 0 || (int64_t)n_sel > (int64_t)r.h_out * r.w_out)
        return fail(VAR_ERR_INDEX, "n_sel=%d outside [0, h*w of the step]", n_sel);
    if (n_sel == 0)   // nothing to attend: every row comes from the base
        return hip_status(varattn::launch_scatter(r, reinterpret_cast<hipStream_t>(stream)),
                          "var_attn_block_sparse_restore launch");
    if (!q_index) return fail(VAR_ERR_NULL, "q_index must be non-NULL when n_sel > 0");
    return sparse_impl(sched, desc, q, q_l, k, k_l, v, v_l, o, o_l, lse, q_index, n_sel, row_ptr, col_idx, tile_q,
                       tile_k, 1, nullptr, 0, stream, -1, nullptr, &r);
}

VAR_EXPORT var_status var_attn_block_sparse_heads(const var_schedule* sched, const var_attn_desc* desc,
                                                  const void* q, var_layout q_l, const void* k, var_layout k_l,
                                                  const void* v, var_layout v_l, void* o, var_layout o_l,
                                                  float* lse, const int32_t* q_index, int32_t n_sel,
                                                  const int32_t* row_ptr, const int32_t* col_idx,
                                                  int64_t col_stride, void* stream) {
    if (col_stride < 0) return fail(VAR_ERR_RANGE, "col_stride must be >= 0");
    return sparse_impl(sched, desc, q, q_l, k, k_l, v, v_l, o, o_l, lse, q_index, n_sel, row_ptr, col_idx, 64, 64, 1,
                       nullptr, 0, stream, col_stride);
}

VAR_EXPORT var_status var_attn_dense_e4m3(const var_schedule* sched, const var_attn_desc* desc, const void* q,
                                          var_layout q_l, const uint8_t* k, var_layout k_l, const float* k_scale,
                                          int64_t k_scale_stride, const void* v, var_layout v_l, void* o,
                                          var_layout o_l, float* lse, const int32_t* q_index, int32_t n_sel,
                                          int32_t n_splits, void* workspace, int64_t workspace_bytes,
                                          void* stream) {
    const E4m3Keys kc{k_scale, k_scale_stride};
    return dense_impl(sched, desc, q, q_l, k, k_l, v, v_l, o, o_l, lse, q_index, n_sel, n_splits, workspace,
                      workspace_bytes, stream, &kc);
}

VAR_EXPORT var_status var_attn_block_sparse_e4m3(const var_schedule* sched, const var_attn_desc* desc,
                                                 const void* q, var_layout q_l, const uint8_t* k, var_layout k_l,
                                                 const float* k_scale, int64_t k_scale_stride, const void* v,
                                                 var_layout v_l, void* o, var_layout o_l, float* lse,
                                                 const int32_t* q_index, int32_t n_sel, const int32_t* row_ptr,
                                                 const int32_t* col_idx, int64_t col_stride, void* stream) {
    if (col_stride < 0) return fail(VAR_ERR_RANGE, "col_stride must be >= 0");
    const E4m3Keys kc{k_scale, k_scale_stride};
    return sparse_impl(sched, desc, q, q_l, k, k_l, v, v_l, o, o_l, lse, q_index, n_sel, row_ptr, col_idx, 64, 64, 1,
                       nullptr, 0, stream, col_stride > 0 ? col_stride : -1, &kc);
}

VAR_EXPORT var_status var_quantize_e4m3(int32_t batch, int32_t heads, int32_t tokens, int32_t head_dim,
                                        const void* x, var_layout x_l, uint8_t* codes, var_layout c_l, float* scale,
                                        int64_t scale_stride, int32_t first_token, void* stream) {
    if (batch < 1 || heads < 1 || (int64_t)batch * heads > 65535)
        return fail(VAR_ERR_RANGE, "batch=%d heads=%d invalid (at most 65535 maps)", batch, heads);
    if (tokens < 0 || tokens >= (1 << 24)) return fail(VAR_ERR_RANGE, "tokens=%d outside [0, 2^24)", tokens);
    if (first_token < 0 || first_token > tokens)
        return fail(VAR_ERR_RANGE, "first_token=%d outside [0, tokens=%d]", first_token, tokens);
    if (head_dim < 16 || head_dim > 256 || head_dim % 16)
        return fail(VAR_ERR_UNSUPPORTED, "head_dim=%d must be a multiple of 16 in [16, 256]", head_dim);
    const int32_t n_tiles = (tokens + 63) / 64;
    if (first_token == tokens) return ok();   // no tile to write
    if (!x || !codes || !scale) return fail(VAR_ERR_NULL, "x, codes and scale must be non-NULL");
    if (!aligned16(x) || !aligned16(codes)) return fail(VAR_ERR_STRIDE, "x and codes must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(scale) & 3u) return fail(VAR_ERR_STRIDE, "scale must be 4-byte aligned");
    if (scale_stride < n_tiles)
        return fail(VAR_ERR_STRIDE, "scale_stride=%lld below the %d tiles", (long long)scale_stride, n_tiles);
    var_status st = check_layout("x", x_l, head_dim, 2);
    if (st != VAR_OK) return st;
    if ((st = check_layout("codes", c_l, head_dim, 1)) != VAR_OK) return st;
    varattn::QuantParams p;
    std::memset(&p, 0, sizeof(p));
    p.x = x;
    p.codes = codes;
    p.scale = scale;
    p.scale_stride = scale_stride;
    p.x_sb = x_l.batch; p.x_sh = x_l.head; p.x_st = x_l.token;
    p.c_sb = c_l.batch; p.c_sh = c_l.head; p.c_st = c_l.token;
    p.H = heads;
    p.maps = batch * heads;
    p.tokens = tokens;
    p.D = head_dim;
    p.tile_first = first_token / 64;
    return hip_status(varattn::launch_quant_e4m3(p, reinterpret_cast<hipStream_t>(stream)),
                      "var_quantize_e4m3 launch");
}

VAR_EXPORT var_status var_attn_block_mass(const var_schedule* sched, const var_attn_desc* d, const void* q,
                                          var_layout q_l, const void* k, var_layout k_l, const float* lse,
                                          float* mass, void* stream) {
    Offsets off;
    var_status st = check_schedule(sched, &off);
    if (st != VAR_OK) return st;
    if (!d) return fail(VAR_ERR_NULL, "desc is NULL");
    if ((st = check_range(off, d->q_scale_begin, d->q_scale_end)) != VAR_OK) return st;
    if (d->q_scale_end != d->q_scale_begin + 1)
        return fail(VAR_ERR_RANGE, "block mass takes one scale, got [%d, %d)", d->q_scale_begin, d->q_scale_end);
    if (d->batch < 1 || d->heads < 1 || (int64_t)d->batch * d->heads > (1 << 20))
        return fail(VAR_ERR_RANGE, "batch=%d heads=%d invalid", d->batch, d->heads);
    if (d->in_dtype != VAR_BF16 || (d->head_dim != 64 && d->head_dim != 128))
        return fail(VAR_ERR_UNSUPPORTED, "block mass supports bf16 input with head_dim 64 or 128");
    if (!(d->softmax_scale >= 0.f) || std::isinf(d->softmax_scale))
        return fail(VAR_ERR_RANGE, "softmax_scale must be finite and >= 0 (0 = 1/sqrt(D))");
    const int32_t n = off.off[d->q_scale_end] - off.off[d->q_scale_begin];
    const int32_t L = off.off[d->q_scale_end];
    if (n > varattn::kMassMaxRows)
        return fail(VAR_ERR_UNSUPPORTED, "decision step of %d rows above %d", n, varattn::kMassMaxRows);
    if (!q || !k || !lse || !mass) return fail(VAR_ERR_NULL, "q, k, lse and mass must be non-NULL");
    if (!aligned16(q) || !aligned16(k)) return fail(VAR_ERR_STRIDE, "q and k must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(mass) & 3u))
        return fail(VAR_ERR_STRIDE, "lse and mass must be 4-byte aligned");
    if ((st = check_layout("q", q_l, d->head_dim, 2)) != VAR_OK) return st;
    if ((st = check_layout("k", k_l, d->head_dim, 2)) != VAR_OK) return st;
    varattn::MassParams p;
    std::memset(&p, 0, sizeof(p));
    p.q = q;
    p.k = k;
    p.lse = lse;
    p.mass = mass;
    p.q_sb = q_l.batch; p.q_sh = q_l.head; p.q_st = q_l.token;
    p.k_sb = k_l.batch; p.k_sh = k_l.head; p.k_st = k_l.token;
    p.B = d->batch;
    p.H = d->heads;
    p.n_rows = n;
    p.kv_len = L;
    p.n_kt = (L + 63) / 64;
    if ((int64_t)p.B * p.H * p.n_kt >= ((int64_t)1 << 31)) return fail(VAR_ERR_RANGE, "block mass grid too large");
    const float scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / std::sqrt((float)d->head_dim);
    p.scale_log2 = scale * 1.4426950408889634f;
    return hip_status(varattn::launch_block_mass(p, d->head_dim, reinterpret_cast<hipStream_t>(stream)),
                      "var_attn_block_mass launch");
}

VAR_EXPORT var_status var_decision_tiles(int32_t maps, int32_t n_qt, int32_t n_kt, const float* mass, float tau,
                                         uint8_t* kept, void* stream) {
    if (maps < 1 || n_qt < 1 || n_kt < 1 || (int64_t)maps * n_qt >= ((int64_t)1 << 31))
        return fail(VAR_ERR_RANGE, "maps=%d n_qt=%d n_kt=%d invalid", maps, n_qt, n_kt);
    if (n_kt > varattn::kDecisionMaxTiles)
        return fail(VAR_ERR_UNSUPPORTED, "n_kt=%d above %d", n_kt, varattn::kDecisionMaxTiles);
    if (!(tau >= 0.f && tau <= 1.f)) return fail(VAR_ERR_RANGE, "tau must lie in [0, 1]");
    if (!mass || !kept) return fail(VAR_ERR_NULL, "mass and kept must be non-NULL");
    if (reinterpret_cast<uintptr_t>(mass) & 3u) return fail(VAR_ERR_STRIDE, "mass must be 4-byte aligned");
    varattn::DecisionParams p;
    p.mass = mass;
    p.kept = kept;
    p.n_kt = n_kt;
    p.tau = tau;
    return hip_status(varattn::launch_decision(p, maps * n_qt, reinterpret_cast<hipStream_t>(stream)),
                      "var_decision_tiles launch");
}

VAR_EXPORT var_status var_mapped_tile_mask(const var_schedule* sched, int32_t decision_scale, int32_t step,
                                           int32_t maps, const uint8_t* kept_d, int32_t* row_ptr, int32_t* col_idx,
                                           int64_t col_stride, void* stream) {
    Offsets off;
    var_status st = check_schedule(sched, &off);
    if (st != VAR_OK) return st;
    if (decision_scale < 0 || step < decision_scale || step >= off.num_scales)
        return fail(VAR_ERR_RANGE, "need 0 <= decision_scale <= step < num_scales, got %d, %d", decision_scale, step);
    if (maps < 1 || maps > (1 << 20)) return fail(VAR_ERR_RANGE, "maps=%d invalid", maps);
    const int32_t n_d = off.off[decision_scale + 1] - off.off[decision_scale];
    const int32_t n_qt_d = (n_d + 63) / 64, n_kt_d = (off.off[decision_scale + 1] + 63) / 64;
    const int32_t n_t = off.off[step + 1] - off.off[step];
    const int32_t n_qt = (n_t + 63) / 64, n_kt = (off.off[step + 1] + 63) / 64;
    if (n_qt_d > varattn::kDecisionMaxRowTiles || n_kt_d > varattn::kDecisionMaxTiles || n_kt > varattn::kMappedMaxTiles)
        return fail(VAR_ERR_UNSUPPORTED, "decision step %d or step %d too large for the mapped mask", decision_scale,
                    step);
    if (col_stride < (int64_t)n_qt * n_kt)
        return fail(VAR_ERR_CAPACITY, "col_stride=%lld below n_qt*n_kt=%lld", (long long)col_stride,
                    (long long)n_qt * n_kt);
    if ((int64_t)maps * n_qt >= ((int64_t)1 << 31)) return fail(VAR_ERR_RANGE, "mapped mask grid too large");
    if (!kept_d || !row_ptr || !col_idx) return fail(VAR_ERR_NULL, "kept_d, row_ptr and col_idx must be non-NULL");
    varattn::MappedParams p;
    std::memset(&p, 0, sizeof(p));
    p.kept_d = kept_d;
    p.row_ptr = row_ptr;
    p.col_idx = col_idx;
    p.rp_map_stride = n_qt + 1;
    p.ci_map_stride = col_stride;
    p.d = decision_scale;
    p.T = step;
    p.n_qt = n_qt;
    p.n_kt = n_kt;
    p.n_qt_d = n_qt_d;
    p.n_kt_d = n_kt_d;
    for (int i = 0; i <= VAR_MAX_SCALES; ++i) p.off[i] = i <= off.num_scales ? off.off[i] : off.off[off.num_scales];
    for (int i = 0; i < VAR_MAX_SCALES; ++i) {
        p.h[i] = i < off.num_scales ? sched->h[i] : 1;
        p.w[i] = i < off.num_scales ? sched->w[i] : 1;
    }
    return hip_status(varattn::launch_mapped_mask(p, maps, reinterpret_cast<hipStream_t>(stream)),
                      "var_mapped_tile_mask launch");
}

VAR_EXPORT var_status var_attn_split_plan(const var_schedule* sched, const var_attn_desc* d, int32_t n_sel,
                                          int32_t kv_tiles_hint, int32_t* n_splits, int64_t* workspace_bytes) {
    Offsets off;
    var_status st = check_schedule(sched, &off);
    if (st != VAR_OK) return st;
    if (!d) return fail(VAR_ERR_NULL, "desc is NULL");
    if ((st = check_range(off, d->q_scale_begin, d->q_scale_end)) != VAR_OK) return st;
    if (d->batch < 1 || d->heads < 1 || (int64_t)d->batch * d->heads > (1 << 20))
        return fail(VAR_ERR_RANGE, "batch=%d heads=%d invalid", d->batch, d->heads);
    if (d->head_dim < 1) return fail(VAR_ERR_RANGE, "head_dim=%d invalid", d->head_dim);
    const int32_t n_q = off.off[d->q_scale_end] - off.off[d->q_scale_begin];
    if (n_sel < 0 || n_sel > n_q) return fail(VAR_ERR_INDEX, "n_sel=%d outside [0, n_q=%d]", n_sel, n_q);
    if (kv_tiles_hint < 0) return fail(VAR_ERR_RANGE, "kv_tiles_hint must be >= 0");
    const int64_t rows = n_sel > 0 ? n_sel : n_q;
    const int64_t bh = (int64_t)d->batch * d->heads;
    int32_t s = 1;
    if (d->in_dtype == VAR_BF16) {
        const int cus = device_cu_count();
        const int rpt = varattn::attn_bf16_rows_per_tile(d->head_dim, false, bh, rows, cus);
        const int64_t tasks = bh * ((rows + rpt - 1) / rpt);
        const int64_t tiles = kv_tiles_hint > 0 ? kv_tiles_hint : (off.off[d->q_scale_end] + 63) / 64;
        const int64_t cap =
            (int64_t)cus * varattn::attn_bf16_resident_wgs(d->head_dim, d->out_dtype == VAR_BF16, false, rpt);
        s = choose_splits(tasks, tiles, bh * rows, d->head_dim, cap);
    }
    if (n_splits) *n_splits = s;
    if (workspace_bytes) {
        *workspace_bytes = 0;
        if (s > 1) {   // enough for a dense or a block-sparse call (their work items differ)
            for (const bool sp : {false, true}) {
                const int rpt = varattn::attn_bf16_rows_per_tile(d->head_dim, sp, bh, rows, device_cu_count());
                const int64_t cap = (int64_t)device_cu_count() *
                                    varattn::attn_bf16_resident_wgs(d->head_dim, d->out_dtype == VAR_BF16, sp, rpt);
                const int64_t need = split_need_bytes(s, split_rows(bh, rows, rpt, cap).part_rows, d->head_dim);
                *workspace_bytes = need > *workspace_bytes ? need : *workspace_bytes;
            }
        }
    }
    return ok();
}

VAR_EXPORT var_status var_attn_dense_split(const var_schedule* sched, const var_attn_desc* desc, const void* q,
                                           var_layout q_l, const void* k, var_layout k_l, const void* v,
                                           var_layout v_l, void* o, var_layout o_l, float* lse,
                                           const int32_t* q_index, int32_t n_sel, int32_t n_splits,
                                           void* workspace, int64_t workspace_bytes, void* stream) {
    return dense_impl(sched, desc, q, q_l, k, k_l, v, v_l, o, o_l, lse, q_index, n_sel, n_splits, workspace,
                      workspace_bytes, stream);
}

namespace {

// The split partials of var_attn_dense_split_noalloc: a file-scope device
// array, one copy per device (loaded with the code object), reached from the
// host through its device address, looked up once per device.
constexpr int64_t kScratchBytes = VAR_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

void* scratch_address() {
    constexpr int kMaxDevices = 64;
    static std::atomic<void*> addr[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* ptr = addr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        addr[dev].store(ptr, std::memory_order_release);
    }
    return ptr;
}

}  // namespace

VAR_EXPORT var_status var_attn_dense_split_noalloc(const var_schedule* sched, const var_attn_desc* desc,
                                                   const void* q, var_layout q_l, const void* k, var_layout k_l,
                                                   const void* v, var_layout v_l, void* o, var_layout o_l,
                                                   float* lse, const int32_t* q_index, int32_t n_sel,
                                                   int32_t n_splits, void* stream) {
    if (n_splits == 1)
        return dense_impl(sched, desc, q, q_l, k, k_l, v, v_l, o, o_l, lse, q_index, n_sel, 1, nullptr, 0, stream);
    // the partials this call needs, checked against the scratch before anything
    // is launched (only the device's compute-unit count and occupancy are queried)
    Offsets off;
    var_status st = check_schedule(sched, &off);
    if (st != VAR_OK) return st;
    if (!desc) return fail(VAR_ERR_NULL, "desc is NULL");
    if ((st = check_range(off, desc->q_scale_begin, desc->q_scale_end)) != VAR_OK) return st;
    if (n_splits < 1 || n_splits > varattn::kMaxSplits)
        return fail(VAR_ERR_RANGE, "n_splits=%d outside [1, %d]", n_splits, varattn::kMaxSplits);
    if (desc->in_dtype != VAR_BF16 || (desc->head_dim != 64 && desc->head_dim != 128))
        return fail(VAR_ERR_UNSUPPORTED, "key splits need bf16 input with head_dim 64 or 128");
    if (desc->batch < 1 || desc->heads < 1 || (int64_t)desc->batch * desc->heads > (1 << 20))
        return fail(VAR_ERR_RANGE, "batch=%d heads=%d invalid", desc->batch, desc->heads);
    const int64_t n_q = off.off[desc->q_scale_end] - off.off[desc->q_scale_begin];
    const int64_t rows = q_index ? n_sel : n_q;
    if (rows > 0) {
        const int64_t bh = (int64_t)desc->batch * desc->heads;
        const int rpt = varattn::attn_bf16_rows_per_tile(desc->head_dim, false, bh, rows, device_cu_count());
        const int64_t cap = (int64_t)device_cu_count() *
                            varattn::attn_bf16_resident_wgs(desc->head_dim, desc->out_dtype == VAR_BF16, false, rpt);
        const int64_t need = split_need_bytes(n_splits, split_rows(bh, rows, rpt, cap).part_rows, desc->head_dim);
        if (need > kScratchBytes)
            return fail(VAR_ERR_CAPACITY, "the call needs %lld bytes of split partials, above the library's "
                        "static scratch of %lld bytes (use var_attn_dense_split with a workspace)",
                        (long long)need, (long long)kScratchBytes);
    }
    void* ws = scratch_address();
    if (!ws) return fail(VAR_ERR_HIP, "the address of the static scratch is unavailable on this device");
    return dense_impl(sched, desc, q, q_l, k, k_l, v, v_l, o, o_l, lse, q_index, n_sel, n_splits, ws,
                      kScratchBytes, stream);
}

VAR_EXPORT var_status var_attn_block_sparse_split(const var_schedule* sched, const var_attn_desc* desc,
                                                  const void* q, var_layout q_l, const void* k, var_layout k_l,
                                                  const void* v, var_layout v_l, void* o, var_layout o_l,
                                                  float* lse, const int32_t* q_index, int32_t n_sel,
                                                  const int32_t* row_ptr, const int32_t* col_idx, int32_t tile_q,
                                                  int32_t tile_k, int32_t n_splits, void* workspace,
                                                  int64_t workspace_bytes, void* stream) {
    return sparse_impl(sched, desc, q, q_l, k, k_l, v, v_l, o, o_l, lse, q_index, n_sel, row_ptr, col_idx, tile_q,
                       tile_k, n_splits, workspace, workspace_bytes, stream);
}

namespace {
var_status mask_dims(const var_schedule* sched, int32_t b, int32_t e, const var_mask_params* mp, bool has_index,
                     int32_t n_sel, Offsets* off, int32_t* rows, int32_t* n_qt, int32_t* n_kt) {
    var_status st = check_schedule(sched, off);
    if (st != VAR_OK) return st;
    if ((st = check_range(*off, b, e)) != VAR_OK) return st;
    if (!mp) return fail(VAR_ERR_NULL, "mask params are NULL");
    if (mp->tile_q < 1 || mp->tile_k < 1 || mp->tile_q > 4096 || mp->tile_k > 4096)
        return fail(VAR_ERR_RANGE, "tile sizes %dx%d outside [1, 4096]", mp->tile_q, mp->tile_k);
    if (mp->radius_y < 0 || mp->radius_x < 0 || mp->radius_y > 4096 || mp->radius_x > 4096)
        return fail(VAR_ERR_RANGE, "radii must lie in [0, 4096]");
    if (mp->sink_scales < 0 || mp->local_from_scale < 0)
        return fail(VAR_ERR_RANGE, "sink_scales and local_from_scale must be >= 0");
    const int32_t n_q = off->off[e] - off->off[b];
    if (has_index) {
        if (n_sel < 0 || n_sel > n_q) return fail(VAR_ERR_INDEX, "n_sel=%d outside [0, n_q=%d]", n_sel, n_q);
        *rows = n_sel;
    } else {
        if (n_sel != 0) return fail(VAR_ERR_INDEX, "n_sel=%d given without q_index", n_sel);
        *rows = n_q;
    }
    *n_qt = (*rows + mp->tile_q - 1) / mp->tile_q;
    *n_kt = (off->off[e] + mp->tile_k - 1) / mp->tile_k;
    return VAR_OK;
}
}  // namespace

VAR_EXPORT var_status var_tile_mask_dims(const var_schedule* sched, int32_t b, int32_t e, const var_mask_params* mp,
                                         int32_t n_sel_or_0, int32_t* n_qt, int32_t* n_kt) {
    Offsets off;
    int32_t rows, a, c;
    var_status st = mask_dims(sched, b, e, mp, n_sel_or_0 > 0, n_sel_or_0, &off, &rows, &a, &c);
    if (st != VAR_OK) return st;
    if (n_qt) *n_qt = a;
    if (n_kt) *n_kt = c;
    return ok();
}

VAR_EXPORT var_status var_build_tile_mask(const var_schedule* sched, int32_t b, int32_t e, const var_mask_params* mp,
                                          const int32_t* q_index, int32_t n_sel, int32_t* row_ptr, int32_t* col_idx,
                                          int64_t col_capacity, void* stream) {
    Offsets off;
    int32_t rows, n_qt, n_kt;
    var_status st = mask_dims(sched, b, e, mp, q_index != nullptr, n_sel, &off, &rows, &n_qt, &n_kt);
    if (st != VAR_OK) return st;
    if (!row_ptr || (!col_idx && n_qt > 0)) return fail(VAR_ERR_NULL, "row_ptr and col_idx must be non-NULL");
    if (col_capacity < (int64_t)n_qt * n_kt)
        return fail(VAR_ERR_CAPACITY, "col_capacity=%lld below n_qt*n_kt=%lld", (long long)col_capacity,
                    (long long)n_qt * n_kt);
    if ((int64_t)n_qt * n_kt >= (int64_t)1 << 31) return fail(VAR_ERR_RANGE, "tile mask too large");
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (n_qt == 0) {
        // empty query set: row_ptr = {0}
        return hip_status(varattn::launch_zero_i32(row_ptr, s), "var_build_tile_mask launch");
    }
    varattn::MaskParams p;
    std::memset(&p, 0, sizeof(p));
    p.q_index = q_index;
    p.row_ptr = row_ptr;
    p.col_idx = col_idx;
    p.n_rows = rows;
    p.q_first = off.off[b];
    p.n_q = off.off[e] - off.off[b];
    p.kv_len = off.off[e];
    p.n_qt = n_qt;
    p.n_kt = n_kt;
    p.tile_q = mp->tile_q;
    p.tile_k = mp->tile_k;
    p.sink_scales = mp->sink_scales;
    p.local_from_scale = mp->local_from_scale;
    p.radius_y = mp->radius_y;
    p.radius_x = mp->radius_x;
    p.num_scales = e;
    for (int i = 0; i <= VAR_MAX_SCALES; ++i) p.off[i] = i <= off.num_scales ? off.off[i] : off.off[off.num_scales];
    for (int i = 0; i < VAR_MAX_SCALES; ++i) {
        p.h[i] = i < off.num_scales ? sched->h[i] : 1;
        p.w[i] = i < off.num_scales ? sched->w[i] : 1;
    }
    return hip_status(varattn::launch_tile_mask(p, s), "var_build_tile_mask launch");
}

VAR_EXPORT var_status var_build_tile_masks(const var_schedule* sched, const var_mask_params* mp,
                                           const var_tile_mask_call* calls, int32_t n_calls, void* stream) {
    static_assert(VAR_MAX_MASK_CALLS == varattn::kMaxMaskBatch, "batch capacity");
    if (!calls) return fail(VAR_ERR_NULL, "calls is NULL");
    if (n_calls < 1 || n_calls > VAR_MAX_MASK_CALLS)
        return fail(VAR_ERR_RANGE, "n_calls=%d outside [1, %d]", n_calls, VAR_MAX_MASK_CALLS);
    varattn::MaskBatch bt;
    std::memset(&bt, 0, sizeof(bt));
    Offsets off{};
    int64_t blocks = 0;
    for (int32_t i = 0; i < n_calls; ++i) {
        const var_tile_mask_call& c = calls[i];
        int32_t rows, n_qt, n_kt;
        var_status st = mask_dims(sched, c.q_scale_begin, c.q_scale_end, mp, c.q_index != nullptr, c.n_sel, &off,
                                  &rows, &n_qt, &n_kt);
        if (st != VAR_OK) {
            char msg[256];
            std::snprintf(msg, sizeof(msg), "%s", var_last_error());   // (fail rewrites the same buffer)
            return fail(st, "call %d: %s", i, msg);
        }
        if (!c.row_ptr || (!c.col_idx && n_qt > 0))
            return fail(VAR_ERR_NULL, "call %d: row_ptr and col_idx must be non-NULL", i);
        if (c.col_capacity < (int64_t)n_qt * n_kt)
            return fail(VAR_ERR_CAPACITY, "call %d: col_capacity=%lld below n_qt*n_kt=%lld", i,
                        (long long)c.col_capacity, (long long)n_qt * n_kt);
        if ((int64_t)n_qt * n_kt >= (int64_t)1 << 31) return fail(VAR_ERR_RANGE, "call %d: tile mask too large", i);
        varattn::MaskCall& m = bt.c[i];
        m.q_index = c.q_index;
        m.row_ptr = c.row_ptr;
        m.col_idx = c.col_idx;
        m.n_rows = rows;
        m.q_first = off.off[c.q_scale_begin];
        m.n_q = off.off[c.q_scale_end] - off.off[c.q_scale_begin];
        m.kv_len = off.off[c.q_scale_end];
        m.n_qt = n_qt;
        m.n_kt = n_kt;
        m.num_scales = c.q_scale_end;
        bt.first_block[i] = (int32_t)blocks;
        blocks += n_qt;
        if (blocks >= ((int64_t)1 << 31)) return fail(VAR_ERR_RANGE, "too many query tiles in the batch");
    }
    bt.first_block[n_calls] = (int32_t)blocks;
    for (int32_t i = n_calls + 1; i <= varattn::kMaxMaskBatch; ++i) bt.first_block[i] = (int32_t)blocks;
    bt.n_calls = n_calls;
    bt.tile_q = mp->tile_q;
    bt.tile_k = mp->tile_k;
    bt.sink_scales = mp->sink_scales;
    bt.local_from_scale = mp->local_from_scale;
    bt.radius_y = mp->radius_y;
    bt.radius_x = mp->radius_x;
    for (int i = 0; i <= VAR_MAX_SCALES; ++i) bt.off[i] = i <= off.num_scales ? off.off[i] : off.off[off.num_scales];
    for (int i = 0; i < VAR_MAX_SCALES; ++i) {
        bt.h[i] = i < off.num_scales ? sched->h[i] : 1;
        bt.w[i] = i < off.num_scales ? sched->w[i] : 1;
    }
    return hip_status(varattn::launch_tile_mask_batch(bt, reinterpret_cast<hipStream_t>(stream)),
                      "var_build_tile_masks launch");
}

VAR_EXPORT var_status var_attn_saliency(const var_schedule* sched, const var_attn_desc* d, const void* q,
                                        var_layout q_l, const void* k, var_layout k_l, const float* lse,
                                        float* saliency, void* stream) {
    Offsets off;
    var_status st = check_schedule(sched, &off);
    if (st != VAR_OK) return st;
    if (!d) return fail(VAR_ERR_NULL, "desc is NULL");
    if ((st = check_range(off, d->q_scale_begin, d->q_scale_end)) != VAR_OK) return st;
    if (d->q_scale_end != d->q_scale_begin + 1)
        return fail(VAR_ERR_RANGE, "saliency takes one scale, got [%d, %d)", d->q_scale_begin, d->q_scale_end);
    if (d->batch < 1 || d->heads < 1 || (int64_t)d->batch * d->heads > (1 << 20))
        return fail(VAR_ERR_RANGE, "batch=%d heads=%d invalid", d->batch, d->heads);
    if (d->in_dtype != VAR_BF16 || (d->head_dim != 64 && d->head_dim != 128))
        return fail(VAR_ERR_UNSUPPORTED, "saliency supports bf16 input with head_dim 64 or 128");
    if (!(d->softmax_scale >= 0.f) || std::isinf(d->softmax_scale))
        return fail(VAR_ERR_RANGE, "softmax_scale must be finite and >= 0 (0 = 1/sqrt(D))");
    if (!q || !k || !lse || !saliency) return fail(VAR_ERR_NULL, "q, k, lse and saliency must be non-NULL");
    if (!aligned16(q) || !aligned16(k)) return fail(VAR_ERR_STRIDE, "q and k must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(saliency) & 3u))
        return fail(VAR_ERR_STRIDE, "lse and saliency must be 4-byte aligned");
    if ((st = check_layout("q", q_l, d->head_dim, 2)) != VAR_OK) return st;
    if ((st = check_layout("k", k_l, d->head_dim, 2)) != VAR_OK) return st;
    varattn::SaliencyParams p;
    std::memset(&p, 0, sizeof(p));
    p.q = q;
    p.k = k;
    p.lse = lse;
    p.sal = saliency;
    p.q_sb = q_l.batch; p.q_sh = q_l.head; p.q_st = q_l.token;
    p.k_sb = k_l.batch; p.k_sh = k_l.head; p.k_st = k_l.token;
    p.B = d->batch;
    p.H = d->heads;
    p.key_first = off.off[d->q_scale_begin];
    p.n_s = off.off[d->q_scale_end] - p.key_first;
    p.n_kb = (p.n_s + 63) / 64;
    if ((int64_t)p.B * p.H * p.n_kb >= ((int64_t)1 << 31)) return fail(VAR_ERR_RANGE, "saliency grid too large");
    const float scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / std::sqrt((float)d->head_dim);
    p.scale_log2 = scale * 1.4426950408889634f;
    return hip_status(varattn::launch_saliency(p, d->head_dim, reinterpret_cast<hipStream_t>(stream)),
                      "var_attn_saliency launch");
}

VAR_EXPORT var_status var_select_topk(int32_t maps, const float* saliency, int32_t h_src, int32_t w_src,
                                      int32_t h_dst, int32_t w_dst, int32_t n_keep, int32_t* q_index,
                                      void* stream) {
    if (maps < 1 || maps > (1 << 20)) return fail(VAR_ERR_RANGE, "maps=%d outside [1, 2^20]", maps);
    if (h_src < 1 || w_src < 1 || h_dst < 1 || w_dst < 1 || h_src > 4096 || w_src > 4096 || h_dst > 4096 ||
        w_dst > 4096)
        return fail(VAR_ERR_RANGE, "grids %dx%d -> %dx%d outside [1, 4096]", h_src, w_src, h_dst, w_dst);
    if (h_src * w_src > varattn::kSelectMaxSrc)
        return fail(VAR_ERR_UNSUPPORTED, "source grid %dx%d above %d positions", h_src, w_src, varattn::kSelectMaxSrc);
    const int64_t n_dst = (int64_t)h_dst * w_dst;
    if (n_keep < 0 || n_keep > n_dst)
        return fail(VAR_ERR_RANGE, "n_keep=%d outside [0, %lld]", n_keep, (long long)n_dst);
    if (n_keep == 0) return ok();
    if (!saliency || !q_index) return fail(VAR_ERR_NULL, "saliency and q_index must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(saliency) & 3u) || (reinterpret_cast<uintptr_t>(q_index) & 3u))
        return fail(VAR_ERR_STRIDE, "saliency and q_index must be 4-byte aligned");
    varattn::SelectParams p;
    p.sal = saliency;
    p.q_index = q_index;
    p.maps = maps;
    p.h_src = h_src;
    p.w_src = w_src;
    p.h_dst = h_dst;
    p.w_dst = w_dst;
    p.n_keep = n_keep;
    return hip_status(varattn::launch_select_topk(p, reinterpret_cast<hipStream_t>(stream)), "var_select_topk launch");
}

VAR_EXPORT var_status var_scatter_restore(int32_t maps, int32_t row_elems, var_dtype dtype, const void* base,
                                          int64_t base_map_stride, int64_t base_row_stride, int32_t h_in,
                                          int32_t w_in, const void* upd, int64_t upd_map_stride,
                                          int64_t upd_row_stride, const int32_t* q_index, int32_t n_sel, void* out,
                                          int64_t out_map_stride, int64_t out_row_stride, int32_t h_out,
                                          int32_t w_out, int32_t* err_flag, void* stream) {
    if (dtype != VAR_F32 && dtype != VAR_BF16) return fail(VAR_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    if (maps < 0 || row_elems < 1) return fail(VAR_ERR_RANGE, "maps=%d row_elems=%d invalid", maps, row_elems);
    if (h_in < 1 || w_in < 1 || h_out < 1 || w_out < 1 || (int64_t)h_in * w_in >= kMaxTokens ||
        (int64_t)h_out * w_out >= kMaxTokens)
        return fail(VAR_ERR_RANGE, "grid sizes invalid");
    if (n_sel < 0 || (int64_t)n_sel > (int64_t)h_out * w_out)
        return fail(VAR_ERR_INDEX, "n_sel=%d outside [0, h_out*w_out]", n_sel);
    if (!base || !out || (n_sel > 0 && !q_index))
        return fail(VAR_ERR_NULL, "base, out (and q_index when n_sel > 0) must be non-NULL");
    const int eb = dtype == VAR_BF16 ? 2 : 4;
    const int64_t strides[6] = {base_map_stride, base_row_stride, upd_map_stride, upd_row_stride, out_map_stride,
                                out_row_stride};
    for (int i = 0; i < 6; ++i)
        if (strides[i] < 0) return fail(VAR_ERR_STRIDE, "strides must be non-negative");
    if (base_row_stride < row_elems || out_row_stride < row_elems || (n_sel > 0 && upd && upd_row_stride < row_elems))
        return fail(VAR_ERR_STRIDE, "row strides must be >= row_elems");
    if (maps == 0) return ok();
    varattn::ScatterParams p;
    std::memset(&p, 0, sizeof(p));
    p.base = static_cast<const unsigned char*>(base);
    p.upd = static_cast<const unsigned char*>(upd);
    p.out = static_cast<unsigned char*>(out);
    p.q_index = q_index;
    p.err_flag = err_flag;
    p.base_map_stride = base_map_stride * eb;
    p.base_row_stride = base_row_stride * eb;
    p.upd_map_stride = upd_map_stride * eb;
    p.upd_row_stride = upd_row_stride * eb;
    p.out_map_stride = out_map_stride * eb;
    p.out_row_stride = out_row_stride * eb;
    p.maps = maps;
    p.row_bytes = row_elems * eb;
    p.n_sel = n_sel;
    p.h_in = h_in; p.w_in = w_in; p.h_out = h_out; p.w_out = w_out;
    // widest copy unit dividing every byte offset the kernel forms
    uint64_t g = (uint64_t)p.row_bytes | (uint64_t)reinterpret_cast<uintptr_t>(base) |
                 (uint64_t)reinterpret_cast<uintptr_t>(out);
    if (n_sel > 0) g |= (uint64_t)reinterpret_cast<uintptr_t>(upd) | (uint64_t)p.upd_map_stride | (uint64_t)p.upd_row_stride;
    g |= (uint64_t)p.base_map_stride | (uint64_t)p.base_row_stride | (uint64_t)p.out_map_stride |
         (uint64_t)p.out_row_stride;
    p.unit = (g & 15u) == 0 ? 16 : ((g & 3u) == 0 ? 4 : 2);
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return hip_status(varattn::launch_scatter(p, s), "var_scatter_restore launch");
}
