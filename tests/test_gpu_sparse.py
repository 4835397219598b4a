"""GPU parity of the tile-mask builder, the block-sparse kernel and the scatter.

CSR and scatter outputs are compared bit for bit with the oracle; attention
within the bf16 tolerances (max-abs 1e-2, mean-abs 1e-3) or 1e-5 for fp32.
"""

import numpy as np
import pytest
import torch

import oracle
from scale_wise_attention_amd.inputs import WORKLOADS, make_qkv, pruned_index, normal_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from scale_wise_attention_amd import api as _api
    return _api


def _np(t):
    return t.detach().float().cpu().numpy()


def _csr_host(row_ptr, col_idx):
    rp = row_ptr.cpu().numpy()
    return rp, col_idx.cpu().numpy()[: rp[-1]]


def _check(got, ref, tol_max=1e-2, tol_mean=1e-3, what=""):
    err = np.abs(got.astype(np.float64) - ref)
    print(f"[{what}] max-abs {err.max():.3e} mean-abs {err.mean():.3e}", flush=True)
    assert err.max() <= tol_max and err.mean() <= tol_mean, what


def _gpu_mask(api, h, w, qb, qe, tq, tk, sink, local, ry, rx, q_index=None):
    mp = api.mask_params(tq, tk, sink, local, ry, rx)
    idx = None if q_index is None else torch.from_numpy(np.asarray(q_index, np.int32)).cuda()
    rp, ci = api.var_build_tile_mask((h, w), qb, qe, mp, q_index=idx)
    torch.cuda.synchronize()
    return _csr_host(rp, ci)


def _assert_mask_equal(api, h, w, qb, qe, tq, tk, sink, local, ry, rx, q_index=None, what=""):
    rp, ci = _gpu_mask(api, h, w, qb, qe, tq, tk, sink, local, ry, rx, q_index)
    kept = oracle.tile_mask(h, w, qb, qe, tq, tk, sink, local, ry, rx, q_index=q_index)
    erp, eci = oracle.mask_to_csr(kept)
    print(f"[mask {what}] nnz gpu {rp[-1]} oracle {erp[-1]}", flush=True)
    assert np.array_equal(rp, erp), what
    assert np.array_equal(ci, eci), what


def test_mask_tiny_hand_case(api):
    _assert_mask_equal(api, [1, 2, 3, 4], [1, 2, 3, 4], 0, 4, 4, 4, 1, 1, 0, 0, what="tiny")


def test_mask_1024_every_step_and_full_sequence(api):
    wl = WORKLOADS["var1024_sparse"]
    for s in range(wl.num_scales):
        _assert_mask_equal(api, wl.h, wl.w, s, s + 1, 64, 64, 7, 7, 2, 2, what=f"1024 step {s}")
    _assert_mask_equal(api, wl.h, wl.w, 0, wl.num_scales, 64, 64, 7, 7, 2, 2, what="1024 full sequence")


def test_mask_1024_pruned_last_step(api):
    wl = WORKLOADS["var1024_sparse"]
    K = wl.num_scales
    for seed in (0, 1, 2):
        sel = pruned_index(4096, 0.4, seed)
        _assert_mask_equal(api, wl.h, wl.w, K - 1, K, 64, 64, 7, 7, 2, 2, q_index=sel, what=f"pruned seed {seed}")


@pytest.mark.parametrize("tk,sink,local", [(1, 7, 7), (1, 13, 13), (3, 2, 9)])
def test_mask_1024_last_step_many_key_tiles(api, tk, sink, local):
    # more than 8192 key tiles: the builder's bitmap takes several passes
    wl = WORKLOADS["var1024_sparse"]
    K = wl.num_scales
    _assert_mask_equal(api, wl.h, wl.w, K - 1, K, 256, tk, sink, local, 2, 2, what=f"tile_k {tk} sink {sink}")


def test_mask_1024_full_sequence_many_query_tiles(api):
    # more than 8192 query tiles: the compaction moves row by row
    wl = WORKLOADS["var1024_sparse"]
    _assert_mask_equal(api, wl.h, wl.w, 0, wl.num_scales, 1, 64, 7, 7, 2, 2, what="tile_q 1")


@pytest.mark.parametrize("seed", range(24))
def test_mask_random_schedules_and_params(api, seed):
    rng = np.random.default_rng(1000 + seed)
    K = int(rng.integers(1, 7))
    h = [int(a) for a in rng.integers(1, 12, K)]
    w = [int(a) for a in rng.integers(1, 12, K)]
    qb = int(rng.integers(0, K))
    qe = int(rng.integers(qb + 1, K + 1))
    tq, tk = int(rng.integers(1, 20)), int(rng.integers(1, 20))
    sink, local = int(rng.integers(0, K + 1)), int(rng.integers(0, K + 1))
    ry, rx = int(rng.integers(0, 4)), int(rng.integers(0, 4))
    off = oracle.offsets(h, w)
    n_q = off[qe] - off[qb]
    sel = None
    if seed % 2:
        sel = np.sort(rng.choice(n_q, int(rng.integers(1, n_q + 1)), replace=False)).astype(np.int32)
    _assert_mask_equal(api, h, w, qb, qe, tq, tk, sink, local, ry, rx, q_index=sel, what=f"random {seed}")


def test_mask_capacity_error(api):
    wl = WORKLOADS["var1024_sparse"]
    mp = api.mask_params()
    rp = torch.empty(65, dtype=torch.int32, device="cuda")
    ci = torch.empty(100, dtype=torch.int32, device="cuda")
    with pytest.raises(api.VarAttnError) as e:
        api.var_build_tile_mask((wl.h, wl.w), 12, 13, mp, row_ptr=rp, col_idx=ci)
    assert e.value.status_name == "VAR_ERR_CAPACITY"


def _sparse_vs_oracle(api, wl, q, k, v, s, sel=None, rows=None, heads=None, what=""):
    off = oracle.offsets(wl.h, wl.w)
    qs = q[:, :, off[s]:off[s + 1]]
    idx = None if sel is None else torch.from_numpy(sel).cuda()
    mp = api.mask_params(64, 64, wl.sink_scales, wl.local_from_scale, wl.radius, wl.radius)
    rp, ci = api.var_build_tile_mask((wl.h, wl.w), s, s + 1, mp, q_index=idx)
    o = api.var_attn_block_sparse((wl.h, wl.w), qs, k, v, s, s + 1, rp, ci, q_index=idx)
    kept = oracle.tile_mask(wl.h, wl.w, s, s + 1, 64, 64, wl.sink_scales, wl.local_from_scale, wl.radius,
                            wl.radius, q_index=sel)
    on, qn, kn, vn = _np(o), _np(qs), _np(k), _np(v)
    heads = heads or [(b, h) for b in range(q.shape[0]) for h in range(q.shape[1])]
    for (b, h) in heads:
        ref = oracle.attention(qn[b:b + 1, h:h + 1], kn[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1], wl.h, wl.w,
                               s, s + 1, q_index=sel, kept=kept, rows=rows)
        got = on[b:b + 1, h:h + 1] if rows is None else on[b:b + 1, h:h + 1, rows]
        _check(got, ref, what=f"{what} b{b} h{h}")
    return o


def test_sparse_1024_last_step_full_size(api):
    wl = WORKLOADS["var1024_sparse"]
    q, k, v = make_qkv(wl, 0, device="cuda")
    rows = np.unique(np.concatenate([np.arange(0, 4096, 37), [63, 64, 127, 128, 4095]]))
    _sparse_vs_oracle(api, wl, q, k, v, wl.num_scales - 1, rows=rows,
                      heads=[(0, 0), (0, 9), (1, 4), (1, 15)], what="sparse last step")


def test_sparse_1024_pruned_last_step(api):
    wl = WORKLOADS["var1024_sparse"]
    q, k, v = make_qkv(wl, 1, device="cuda")
    sel = pruned_index(4096, 0.4, 1)
    _sparse_vs_oracle(api, wl, q, k, v, wl.num_scales - 1, sel=sel, heads=[(0, 2), (1, 11)], what="sparse pruned")


def test_sparse_1024_middle_steps_one_head(api):
    wl = WORKLOADS["var1024_sparse"]
    q, k, v = make_qkv(wl, 2, device="cuda")
    for s in (6, 8, 10, 11):
        _sparse_vs_oracle(api, wl, q, k, v, s, heads=[(1, 1)], what=f"sparse step {s}")


def test_sparse_all_tiles_kept_equals_dense(api):
    wl = WORKLOADS["var512"]
    q, k, v = make_qkv(wl, 0, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    s = wl.num_scales - 1
    qs = q[:, :, off[s]:]
    n_q, L = off[s + 1] - off[s], off[s + 1]
    n_qt, n_kt = -(-n_q // 64), -(-L // 64)
    rp = torch.arange(0, (n_qt + 1) * n_kt, n_kt, dtype=torch.int32, device="cuda")
    ci = torch.arange(n_kt, dtype=torch.int32, device="cuda").repeat(n_qt)
    dense = api.var_attn_dense((wl.h, wl.w), qs, k, v, s, s + 1)
    sparse = api.var_attn_block_sparse((wl.h, wl.w), qs, k, v, s, s + 1, rp, ci)
    # same tiles in the same order, same 32-row wave groups: bit-identical
    assert torch.equal(dense, sparse)


def test_sparse_fp32_tiny(api):
    wl = WORKLOADS["tiny_fp32"]
    q, k, v = make_qkv(wl, 0, device="cuda")
    rp, ci = api.var_build_tile_mask((wl.h, wl.w), 0, 4, api.mask_params(64, 64, 1, 1, 0, 0))
    o = api.var_attn_block_sparse((wl.h, wl.w), q, k, v, 0, 4, rp, ci)
    kept = oracle.tile_mask(wl.h, wl.w, 0, 4, 64, 64, 1, 1, 0, 0)
    ref = oracle.attention(_np(q), _np(k), _np(v), wl.h, wl.w, 0, 4, kept=kept)
    _check(_np(o), ref, 1e-5, 1e-5, "fp32 sparse")


def test_sparse_empty_rows_give_zero_and_neg_inf_lse(api):
    wl = WORKLOADS["var256"]
    q, k, v = make_qkv(wl, 0, device="cuda")
    s = wl.num_scales - 1
    rp = torch.zeros(5, dtype=torch.int32, device="cuda")   # 4 query tiles, no kept tile
    ci = torch.zeros(1, dtype=torch.int32, device="cuda")
    o, lse = api.var_attn_block_sparse((wl.h, wl.w), q[:, :, 424:], k, v, s, s + 1, rp, ci, return_lse=True)
    assert torch.count_nonzero(o) == 0 and bool(torch.isneginf(lse).all())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_scatter_restore_bit_exact(api, dtype):
    maps, E = 32, 128
    base = torch.from_numpy(normal_tensor((maps, 48 * 48, E), 0)).to(dtype).cuda()
    sel = pruned_index(4096, 0.4, 0)
    upd = torch.from_numpy(normal_tensor((maps, sel.size, E), 1)).to(dtype).cuda()
    idx = torch.from_numpy(sel).cuda()
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = api.var_scatter_restore(base, 48, 48, upd, idx, 64, 64, err_flag=flag)
    ref = oracle.scatter_restore(base.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).cpu().numpy(),
                                 48, 48, upd.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).cpu().numpy(),
                                 sel, 64, 64)
    got = out.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).cpu().numpy()
    assert np.array_equal(got, ref)
    assert int(flag.item()) == 0


def test_scatter_more_row_groups_than_workgroups(api):
    """260 maps x 256 row groups of 16 rows: more groups than the launch's 65536
    workgroups, so workgroups take a second group (and reset its marks)."""
    maps, E = 260, 128
    base = torch.from_numpy(normal_tensor((maps, 48 * 48, E), 3)).to(torch.bfloat16).cuda()
    sel = pruned_index(4096, 0.4, 1)
    upd = torch.from_numpy(normal_tensor((maps, sel.size, E), 4)).to(torch.bfloat16).cuda()
    out = api.var_scatter_restore(base, 48, 48, upd, torch.from_numpy(sel).cuda(), 64, 64)
    ref = oracle.scatter_restore(base.view(torch.int16).cpu().numpy(), 48, 48, upd.view(torch.int16).cpu().numpy(),
                                 sel, 64, 64)
    assert np.array_equal(out.view(torch.int16).cpu().numpy(), ref)


def test_scatter_edge_cases(api):
    # no index: pure nearest upsampling; odd row widths take the 2-byte path
    for (hi, wi, ho, wo, E) in [(48, 48, 64, 64, 64), (3, 5, 7, 9, 3), (4, 4, 4, 4, 8), (7, 3, 5, 2, 5)]:
        base = torch.from_numpy(normal_tensor((3, hi * wi, E), 2)).to(torch.bfloat16).cuda()
        out = api.var_scatter_restore(base, hi, wi, None, None, ho, wo)
        ref = oracle.scatter_restore(base.view(torch.int16).cpu().numpy(), hi, wi,
                                     np.zeros((3, 0, E), np.int16), np.zeros(0, np.int32), ho, wo)
        assert np.array_equal(out.view(torch.int16).cpu().numpy(), ref)
    # every position retained
    base = torch.randn(2, 4, 8, device="cuda")
    upd = torch.randn(2, 16, 8, device="cuda")
    idx = torch.arange(16, dtype=torch.int32, device="cuda")
    out = api.var_scatter_restore(base, 2, 2, upd, idx, 4, 4)
    assert torch.equal(out, upd)


def test_scatter_flags_bad_indices(api):
    base = torch.randn(2, 16, 8, device="cuda")
    upd = torch.randn(2, 3, 8, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    api.var_scatter_restore(base, 4, 4, upd, torch.tensor([1, 1, 2], dtype=torch.int32, device="cuda"), 4, 4,
                            err_flag=flag)
    assert int(flag.item()) & 2
    flag.zero_()
    api.var_scatter_restore(base, 4, 4, upd, torch.tensor([1, 2, 99], dtype=torch.int32, device="cuda"), 4, 4,
                            err_flag=flag)
    assert int(flag.item()) & 1


def test_pruned_pipeline_end_to_end(api):
    """Mask build -> sparse attention on the retained queries -> scatter over the 48x48 base."""
    wl = WORKLOADS["var1024_sparse"]
    q, k, v = make_qkv(wl, 0, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    K = wl.num_scales
    base = api.var_attn_dense((wl.h, wl.w), q[:, :, off[K - 2]:off[K - 1]], k, v, K - 2, K - 1)
    sel = pruned_index(4096, 0.4, 0)
    idx = torch.from_numpy(sel).cuda()
    mp = api.mask_params()
    rp, ci = api.var_build_tile_mask((wl.h, wl.w), K - 1, K, mp, q_index=idx)
    upd = api.var_attn_block_sparse((wl.h, wl.w), q[:, :, off[K - 1]:], k, v, K - 1, K, rp, ci, q_index=idx)
    out = api.var_scatter_restore(base, 48, 48, upd, idx, 64, 64)
    ref = oracle.scatter_restore(base.view(torch.int32).cpu().numpy(), 48, 48, upd.view(torch.int32).cpu().numpy(),
                                 sel, 64, 64)
    assert np.array_equal(out.view(torch.int32).cpu().numpy(), ref)


def test_sparse_rows_whose_first_tiles_differ(api):
    """Caller CSR in which the waves of a workgroup start on different key tiles:
    a wave's first owned tile comes after the walk's first tile, and a masked
    tail tile comes later.  Each row's reference max must come from its own
    first tile."""
    wl = WORKLOADS["var1024_sparse"]
    q, k, v = make_qkv(wl, 8, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    s = 11
    n = off[s + 1] - off[s]
    n_qt, n_kt = -(-n // 64), -(-off[s + 1] // 64)
    kept = np.zeros((n_qt, n_kt), dtype=bool)
    for r in range(n_qt):
        if r % 2 == 0:
            kept[r, 0:11] = True
        else:
            kept[r, 5 + r % 3:21] = True
            kept[r, 50] = True
        kept[r, n_kt - 1] = True          # the masked tail tile
    rp_h, ci_h = oracle.mask_to_csr(kept)
    rp, ci = torch.from_numpy(rp_h).cuda(), torch.from_numpy(ci_h).cuda()
    qs = q[:, :, off[s]:off[s + 1]]
    o = api.var_attn_block_sparse((wl.h, wl.w), qs, k, v, s, s + 1, rp, ci)
    rows = np.arange(0, n, 29)
    qn, kn, vn = _np(qs), _np(k), _np(v)
    for (b, h) in [(0, 1), (1, 8)]:
        ref = oracle.attention(qn[b:b + 1, h:h + 1], kn[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1], wl.h, wl.w,
                               s, s + 1, kept=kept, rows=rows)
        _check(_np(o[b:b + 1, h:h + 1])[:, :, rows], ref, what=f"first tiles differ b{b} h{h}")
