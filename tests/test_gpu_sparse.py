"""GPU parity of the tile-mask builder, the block-sparse kernel and the scatter.

CSR and scatter outputs are compared bit for bit with the oracle; attention
within the bf16 tolerances (max-abs 1e-2, mean-abs 1e-3) or 1e-5 for fp32.
"""

import numpy as np
import pytest
import torch

import oracle
from _oracle_heads import attention_all_heads
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


def test_batched_masks_equal_oracle_and_single_builds(api):
    """var_build_tile_masks over every step of the 1024px generation, the pruned last
    step, an empty selection and the whole sequence in one call: each CSR bit-exact
    against the oracle and against var_build_tile_mask; then a second batch reusing
    the same buffers (stale contents) with another rule."""
    wl = WORKLOADS["var1024_sparse"]
    K = wl.num_scales
    sel = pruned_index(4096, 0.4, 0)
    idx = torch.from_numpy(sel).cuda()
    empty = torch.empty(0, dtype=torch.int32, device="cuda")
    specs = [(s, s + 1, None) for s in range(K)] + [(K - 1, K, sel), (K - 1, K, np.zeros(0, np.int32)),
                                                   (0, K, None)]
    assert len(specs) == api.MAX_MASK_CALLS
    for sink, local, r in ((7, 7, 2), (3, 9, 1)):
        mp = api.mask_params(64, 64, sink, local, r, r)
        calls = []
        for qb, qe, q in specs:
            qi = None if q is None else (empty if q.size == 0 else idx)
            calls.append((qb, qe, qi))
        if sink == 7:
            got = api.var_build_tile_masks((wl.h, wl.w), mp, calls)
            first = got
        else:   # the same buffers again, holding the first batch's lists
            got = api.var_build_tile_masks((wl.h, wl.w), mp, [c + b for c, b in zip(calls, first)])
        torch.cuda.synchronize()
        for (qb, qe, q), (rp, ci), c in zip(specs, got, calls):
            what = f"batch sink {sink} steps {qb}..{qe} {'pruned' if q is not None and q.size else 'empty' if q is not None else ''}"
            rp_h, ci_h = _csr_host(rp, ci)
            kept = oracle.tile_mask(wl.h, wl.w, qb, qe, 64, 64, sink, local, r, r, q_index=q)
            erp, eci = oracle.mask_to_csr(kept)
            print(f"[{what}] nnz {rp_h[-1]}", flush=True)
            assert np.array_equal(rp_h, erp), what
            assert np.array_equal(ci_h, eci), what
            srp, sci = api.var_build_tile_mask((wl.h, wl.w), qb, qe, mp, q_index=c[2])
            torch.cuda.synchronize()
            srp_h, sci_h = _csr_host(srp, sci)
            assert np.array_equal(rp_h, srp_h) and np.array_equal(ci_h, sci_h), what


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


def _sparse_vs_oracle(api, wl, q, k, v, s, sel=None, rows=None, heads=None, what="", out_dtype=None,
                      planned_splits=False):
    """Block-sparse step s (mask built by the library) against the oracle with the
    oracle's own mask.  Without `heads` and `rows`: every (batch, head) and row.
    planned_splits: the key splits the library plans for the call (as the
    benchmark launches it), over a NaN-filled workspace."""
    off = oracle.offsets(wl.h, wl.w)
    qs = q[:, :, off[s]:off[s + 1]]
    idx = None if sel is None else torch.from_numpy(sel).cuda()
    mp = api.mask_params(64, 64, wl.sink_scales, wl.local_from_scale, wl.radius, wl.radius)
    rp, ci = api.var_build_tile_mask((wl.h, wl.w), s, s + 1, mp, q_index=idx)
    n_splits, ws = 1, None
    if planned_splits:
        rp_h = rp.cpu().numpy()
        hint = max(1, int(round(float(rp_h[-1]) / max(1, rp_h.size - 1))))
        B, H, D = q.shape[0], q.shape[1], q.shape[3]
        n_splits, ws_bytes = api.var_attn_split_plan((wl.h, wl.w), s, s + 1, B, H, D,
                                                     n_sel=0 if sel is None else sel.size, kv_tiles_hint=hint)
        if n_splits > 1:
            ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device="cuda").fill_(float("nan"))
    o = api.var_attn_block_sparse((wl.h, wl.w), qs, k, v, s, s + 1, rp, ci, q_index=idx, out_dtype=out_dtype,
                                  n_splits=n_splits, workspace=ws)
    kept = oracle.tile_mask(wl.h, wl.w, s, s + 1, 64, 64, wl.sink_scales, wl.local_from_scale, wl.radius,
                            wl.radius, q_index=sel)
    on, qn, kn, vn = _np(o), _np(qs), _np(k), _np(v)
    if heads is None and rows is None:
        ref = attention_all_heads(qn, kn, vn, wl.h, wl.w, s, s + 1, q_index=sel, kept=kept)
        _check(on, ref, what=f"{what}, {n_splits} key splits, all (b, h), all rows")
        return o
    heads = heads or [(b, h) for b in range(q.shape[0]) for h in range(q.shape[1])]
    for (b, h) in heads:
        ref = oracle.attention(qn[b:b + 1, h:h + 1], kn[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1], wl.h, wl.w,
                               s, s + 1, q_index=sel, kept=kept, rows=rows)
        got = on[b:b + 1, h:h + 1] if rows is None else on[b:b + 1, h:h + 1, rows]
        _check(got, ref, what=f"{what} b{b} h{h}")
    return o


def test_sparse_1024_last_step_full_size(api):
    """The unpruned block-sparse last step (4096 queries x 10521 keys, 1932 of 10560 tiles)
    as the benchmark launches it (bf16 output): every (batch, head) and row."""
    wl = WORKLOADS["var1024_sparse"]
    q, k, v = make_qkv(wl, 0, device="cuda")
    _sparse_vs_oracle(api, wl, q, k, v, wl.num_scales - 1, what="sparse last step", out_dtype=torch.bfloat16,
                      planned_splits=True)


def test_sparse_1024_pruned_last_step(api):
    """The pruned last step (1638 of 4096 queries gathered, block-sparse) as benchmarked:
    every (batch, head) and row."""
    wl = WORKLOADS["var1024_sparse"]
    q, k, v = make_qkv(wl, 1, device="cuda")
    sel = pruned_index(4096, 0.4, 1)
    _sparse_vs_oracle(api, wl, q, k, v, wl.num_scales - 1, sel=sel, what="sparse pruned",
                      out_dtype=torch.bfloat16, planned_splits=True)


def test_sparse_1024_middle_steps(api):
    """The sparse steps with a partial mask (20x20 .. 48x48) as benchmarked: every (batch,
    head) and row."""
    wl = WORKLOADS["var1024_sparse"]
    q, k, v = make_qkv(wl, 2, device="cuda")
    for s in range(wl.sink_scales, wl.num_scales - 1):
        _sparse_vs_oracle(api, wl, q, k, v, s, what=f"sparse step {s}", out_dtype=torch.bfloat16,
                          planned_splits=True)


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


def _csr_with_repeats(kept, seed):
    """CSR of `kept` with some columns repeated right after themselves (the same kept set)."""
    rng = np.random.default_rng(seed)
    cols = []
    for r in range(kept.shape[0]):
        row = []
        for j, c in enumerate(np.nonzero(kept[r])[0]):
            row += [int(c)] * int(rng.integers(2 if j == 0 else 1, 4))   # each row's first column repeated
        cols.append(row)
    rp = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    ci = np.array(sum(cols, []) or [0], dtype=np.int32)
    assert rp[-1] > int(kept.sum()), "some column is repeated"
    return torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()


@pytest.mark.parametrize("wl_name,in_f32", [("var256", False), ("var512", False), ("tiny_fp32", True)])
def test_sparse_caller_csr_with_repeated_columns(api, wl_name, in_f32):
    """A caller's CSR listing a kept tile several times in a row attends it once: equal to the
    call with the unique list (bit for bit) and to the oracle with the kept set."""
    wl = WORKLOADS[wl_name]
    q, k, v = make_qkv(wl, 9, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    s = wl.num_scales - 1
    qs = q[:, :, off[s]:off[s + 1]]
    n_qt, n_kt = -(-(off[s + 1] - off[s]) // 64), -(-off[s + 1] // 64)
    kept = np.random.default_rng(10).random((n_qt, n_kt)) < 0.6
    kept[:, 0] = True
    rp_u, ci_u = (torch.from_numpy(a).cuda() for a in oracle.mask_to_csr(kept))
    rp_r, ci_r = _csr_with_repeats(kept, 11)
    o_u, l_u = api.var_attn_block_sparse((wl.h, wl.w), qs, k, v, s, s + 1, rp_u, ci_u, return_lse=True)
    o_r, l_r = api.var_attn_block_sparse((wl.h, wl.w), qs, k, v, s, s + 1, rp_r, ci_r, return_lse=True)
    assert torch.equal(o_u, o_r) and torch.equal(l_u, l_r)
    ref = oracle.attention(_np(qs), _np(k), _np(v), wl.h, wl.w, s, s + 1, kept=kept)
    if in_f32:
        _check(_np(o_r), ref, 1e-5, 1e-5, f"{wl_name} repeated columns")
    else:
        _check(_np(o_r), ref, what=f"{wl_name} repeated columns")


def test_sparse_e4m3_and_split_with_repeated_columns(api):
    """The same on the e4m3 and key-split paths (head_dim 128)."""
    from scale_wise_attention_amd.inputs import custom_workload
    wl = custom_workload((1, 2, 4, 6, 8, 12, 16, 20), 2, 2, 128)
    q, k, v = make_qkv(wl, 12, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    s = 7
    qs = q[:, :, off[s]:off[s + 1]]
    n_qt, n_kt = -(-(off[s + 1] - off[s]) // 64), -(-off[s + 1] // 64)
    kept = np.random.default_rng(13).random((n_qt, n_kt)) < 0.5
    kept[:, 0] = True
    rp_u, ci_u = (torch.from_numpy(a).cuda() for a in oracle.mask_to_csr(kept))
    rp_r, ci_r = _csr_with_repeats(kept, 14)
    k8, sk = api.var_quantize_e4m3(k)
    a = api.var_attn_block_sparse_e4m3((wl.h, wl.w), qs, k8, sk, v, s, s + 1, rp_u, ci_u)
    b = api.var_attn_block_sparse_e4m3((wl.h, wl.w), qs, k8, sk, v, s, s + 1, rp_r, ci_r)
    assert torch.equal(a, b)
    n = off[s + 1] - off[s]
    ws = api.split_workspace(3, 2, 2, n, 128)
    a = api.var_attn_block_sparse((wl.h, wl.w), qs, k, v, s, s + 1, rp_u, ci_u, n_splits=3, workspace=ws)
    b = api.var_attn_block_sparse((wl.h, wl.w), qs, k, v, s, s + 1, rp_r, ci_r, n_splits=3, workspace=ws)
    ref = oracle.attention(_np(qs), _np(k), _np(v), wl.h, wl.w, s, s + 1, kept=kept)
    _check(_np(b), ref, what="split x3 repeated columns")
    _check(_np(a), ref, what="split x3 unique columns")


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
    """260 maps x 32 row groups of 128 rows (8320): more groups than the launch's
    8192 workgroups, so workgroups take a second group (and reset its marks)."""
    maps, E = 260, 128
    base = torch.from_numpy(normal_tensor((maps, 48 * 48, E), 3)).to(torch.bfloat16).cuda()
    sel = pruned_index(4096, 0.4, 1)
    upd = torch.from_numpy(normal_tensor((maps, sel.size, E), 4)).to(torch.bfloat16).cuda()
    out = api.var_scatter_restore(base, 48, 48, upd, torch.from_numpy(sel).cuda(), 64, 64)
    ref = oracle.scatter_restore(base.view(torch.int16).cpu().numpy(), 48, 48, upd.view(torch.int16).cpu().numpy(),
                                 sel, 64, 64)
    assert np.array_equal(out.view(torch.int16).cpu().numpy(), ref)


@pytest.mark.parametrize("path", ["short list", "long list"])
def test_scatter_paths_full_and_base_only(api, path):
    """A short index list (1638 of 64x64) and a long one (20000 of 160x160, 42 maps x
    200 row groups of 128 rows, more than the launch's 8192 workgroups).  Full scatter bit-exact
    against the oracle; base-only (upd NULL) leaves the retained rows untouched and
    writes every other row as the oracle."""
    if path == "short list":
        maps, E, hi, ho, n_sel, seed = 32, 128, 48, 64, 1638, 5
    else:
        maps, E, hi, ho, n_sel, seed = 42, 128, 100, 160, 20000, 6
    base = torch.from_numpy(normal_tensor((maps, hi * hi, E), seed)).to(torch.bfloat16).cuda()
    sel = np.sort(np.random.default_rng(seed).choice(ho * ho, n_sel, replace=False)).astype(np.int32)
    upd = torch.from_numpy(normal_tensor((maps, n_sel, E), seed + 1)).to(torch.bfloat16).cuda()
    idx = torch.from_numpy(sel).cuda()
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = api.var_scatter_restore(base, hi, hi, upd, idx, ho, ho, err_flag=flag)
    ref = oracle.scatter_restore(base.view(torch.int16).cpu().numpy(), hi, hi, upd.view(torch.int16).cpu().numpy(),
                                 sel, ho, ho)
    assert np.array_equal(out.view(torch.int16).cpu().numpy(), ref) and int(flag.item()) == 0
    sentinel = torch.full_like(out, float("nan"))
    api.var_scatter_restore(base, hi, hi, None, idx, ho, ho, out=sentinel)
    got = sentinel.view(torch.int16).cpu().numpy()
    keep = np.ones(ho * ho, bool)
    keep[sel] = False
    assert np.array_equal(got[:, keep], ref[:, keep])
    assert np.array_equal(got[:, sel], np.full_like(got[:, sel], torch.tensor(float("nan"), dtype=torch.bfloat16)
                                                     .view(torch.int16).item()))
    bad = idx.clone()
    bad[5] = bad[4]
    flag.zero_()
    api.var_scatter_restore(base, hi, hi, upd, bad, ho, ho, err_flag=flag)
    assert int(flag.item()) & 2


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


@pytest.mark.parametrize("maps", ["all", "two"])
def test_sparse_rows_whose_first_tiles_differ(api, maps):
    """Caller CSR in which the waves of a workgroup start on different key tiles:
    a wave's first owned tile comes after the walk's first tile, and a masked
    tail tile comes later.  Each row's reference max must come from its own
    first tile.  All 32 maps: 576 workgroups, two per compute unit; two maps: 36,
    one per unit with tile pairs once every wave has its reference."""
    wl = WORKLOADS["var1024_sparse"]
    q, k, v = make_qkv(wl, 8, device="cuda")
    if maps == "two":
        q, k, v = q[:1, :2], k[:1, :2], v[:1, :2]
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
    for (b, h) in ([(0, 1), (1, 8)] if maps == "all" else [(0, 0), (0, 1)]):
        ref = oracle.attention(qn[b:b + 1, h:h + 1], kn[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1], wl.h, wl.w,
                               s, s + 1, kept=kept, rows=rows)
        _check(_np(o[b:b + 1, h:h + 1])[:, :, rows], ref, what=f"first tiles differ ({maps}) b{b} h{h}")


def test_pruned_rows_written_in_place_and_base_only_scatter(api):
    """The reconstruction fused into the pruned attention ("ARVAR ...", Key Design 3,
    Eq. (8)-(9)): the attention writes each retained row straight to its place in the
    64x64 grid (out_at_index) and the scatter fills only the other rows from the
    nearest-upsampled base (upd NULL).  In either order the result equals, bit for bit,
    the oracle's reconstruction from the same base and the attention's rows; the
    attention rows themselves equal those of the gathered call."""
    wl = WORKLOADS["var1024_sparse"]
    q, k, v = make_qkv(wl, 3, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    K = wl.num_scales
    sel = pruned_index(4096, 0.4, 3)
    idx = torch.from_numpy(sel).cuda()
    qs = q[:, :, off[K - 1]:]
    mp = api.mask_params()
    rp, ci = api.var_build_tile_mask((wl.h, wl.w), K - 1, K, mp, q_index=idx)
    base = api.var_attn_dense((wl.h, wl.w), q[:, :, off[K - 2]:off[K - 1]], k, v, K - 2, K - 1,
                              out_dtype=torch.bfloat16)
    upd = api.var_attn_block_sparse((wl.h, wl.w), qs, k, v, K - 1, K, rp, ci, q_index=idx, out_dtype=torch.bfloat16)
    ref = oracle.scatter_restore(base.view(torch.int16).cpu().numpy().reshape(32, 2304, 128), 48, 48,
                                 upd.view(torch.int16).cpu().numpy().reshape(32, 1638, 128), sel, 64, 64)
    for order in ("attention first", "scatter first"):
        out = torch.full((2, 16, 4096, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        calls = [lambda: api.var_attn_block_sparse((wl.h, wl.w), qs, k, v, K - 1, K, rp, ci, q_index=idx, out=out,
                                                   out_at_index=True),
                 lambda: api.var_scatter_restore(base, 48, 48, None, idx, 64, 64, out=out)]
        for c in (calls if order == "attention first" else calls[::-1]):
            c()
        got = out.view(torch.int16).cpu().numpy().reshape(32, 4096, 128)
        assert np.array_equal(got, ref), order
    # the same through the dense, key-split and e4m3 kernels: rows land where the gather took them
    out = torch.zeros(2, 16, 4096, 128, dtype=torch.float32, device="cuda")
    api.var_attn_dense((wl.h, wl.w), qs, k, v, K - 1, K, q_index=idx, out=out, out_at_index=True)
    dense_g = api.var_attn_dense((wl.h, wl.w), qs, k, v, K - 1, K, q_index=idx)
    assert torch.equal(out[:, :, idx.long()], dense_g)
    untouched = torch.ones(4096, dtype=torch.bool, device="cuda")
    untouched[idx.long()] = False
    assert int(torch.count_nonzero(out[:, :, untouched])) == 0
    ws = api.split_workspace(3, 2, 16, sel.size, 128)
    out.zero_()
    api.var_attn_dense((wl.h, wl.w), qs, k, v, K - 1, K, q_index=idx, out=out, out_at_index=True, n_splits=3,
                       workspace=ws)
    split_g = api.var_attn_dense((wl.h, wl.w), qs, k, v, K - 1, K, q_index=idx, n_splits=3, workspace=ws)
    assert torch.equal(out[:, :, idx.long()], split_g)
    assert int(torch.count_nonzero(out[:, :, untouched])) == 0
    k8, sk = api.var_quantize_e4m3(k)
    out8 = torch.zeros(2, 16, 4096, 128, dtype=torch.bfloat16, device="cuda")
    api.var_attn_block_sparse_e4m3((wl.h, wl.w), qs, k8, sk, v, K - 1, K, rp, ci, q_index=idx, out=out8,
                                   out_at_index=True)
    g8 = api.var_attn_block_sparse_e4m3((wl.h, wl.w), qs, k8, sk, v, K - 1, K, rp, ci, q_index=idx,
                                        out_dtype=torch.bfloat16)
    assert torch.equal(out8[:, :, idx.long()], g8)


def test_out_at_index_fp32_kernel_and_errors(api):
    wl = WORKLOADS["tiny_fp32"]
    q, k, v = make_qkv(wl, 4, device="cuda")
    sel = np.array([1, 4, 8], np.int32)
    idx = torch.from_numpy(sel).cuda()
    qs = q[:, :, 5:14]
    out = torch.full((1, 2, 9, 32), -7.0, device="cuda")
    api.var_attn_dense((wl.h, wl.w), qs, k, v, 2, 3, q_index=idx, out=out, out_at_index=True)
    g = api.var_attn_dense((wl.h, wl.w), qs, k, v, 2, 3, q_index=idx)
    assert torch.equal(out[:, :, idx.long()], g)
    rest = [i for i in range(9) if i not in sel]
    assert bool((out[:, :, rest] == -7.0).all())
    with pytest.raises(ValueError):
        api.var_attn_dense((wl.h, wl.w), qs, k, v, 2, 3, out_at_index=True)


def _restore_case(api, wl_name, seed, frac, B=None, H=None, out_dtype=torch.bfloat16):
    wl = WORKLOADS[wl_name]
    q, k, v = make_qkv(wl, seed, device="cuda")
    if B is not None:
        q, k, v = q[:B, :H], k[:B, :H], v[:B, :H]
    off = oracle.offsets(wl.h, wl.w)
    K = wl.num_scales
    n = wl.h[-1] * wl.w[-1]
    sel = pruned_index(n, frac, seed) if frac < 1 else np.arange(n, dtype=np.int32)
    idx = torch.from_numpy(np.ascontiguousarray(sel, dtype=np.int32)).cuda()
    qs = q[:, :, off[K - 1]:]
    sink = 7 if wl_name.startswith("var1024") else 3
    mp = api.mask_params(64, 64, sink, sink, 2, 2)
    rp, ci = api.var_build_tile_mask((wl.h, wl.w), K - 1, K, mp, q_index=idx)
    base = api.var_attn_dense((wl.h, wl.w), q[:, :, off[K - 2]:off[K - 1]], k, v, K - 2, K - 1,
                              out_dtype=out_dtype)
    return wl, q, k, v, K, n, sel, idx, qs, rp, ci, base


@pytest.mark.parametrize("wl_name,frac,maps,out_dtype", [
    ("var1024_sparse", 0.4, None, torch.bfloat16),    # 416 attention workgroups, two per compute unit
    ("var1024_sparse", 0.4, None, torch.float32),
    ("var1024_sparse", 0.4, (1, 2), torch.bfloat16),  # a few workgroups: the one-per-unit walk
    ("var1024_sparse", 0.4, (2, 8), torch.bfloat16),  # 208 one-per-unit workgroups: too few free slots, two launches
    ("var1024_sparse", 0.05, None, torch.bfloat16),   # mostly reconstruction
    ("var256", 0.4, None, torch.bfloat16),            # head_dim 64
    ("var256", 1.0, None, torch.float32),             # every row retained: nothing from the base
])
def test_sparse_restore_one_launch(api, wl_name, frac, maps, out_dtype):
    """A pruned step and its reconstruction ("ARVAR ...", Key Design 3, Eq. (8)-(9)) in one
    launch: equal, bit for bit over a NaN-filled output, to the attention writing its rows
    in place followed by the base-only scatter, and to the oracle's reconstruction from the
    same base and the gathered call's rows; the retained rows on a few heads against the
    oracle's attention."""
    B, H = maps if maps else (None, None)
    wl, q, k, v, K, n, sel, idx, qs, rp, ci, base = _restore_case(api, wl_name, 5, frac, B, H, out_dtype)
    Bq, Hq, D = qs.shape[0], qs.shape[1], qs.shape[3]
    hi, wi, ho, wo = wl.h[-2], wl.w[-2], wl.h[-1], wl.w[-1]
    out = torch.full((Bq, Hq, n, D), float("nan"), dtype=out_dtype, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    api.var_attn_block_sparse_restore((wl.h, wl.w), qs, k, v, K - 1, rp, ci, idx, base, hi, wi, out=out,
                                      err_flag=flag)
    two = torch.full_like(out, float("nan"))
    api.var_attn_block_sparse((wl.h, wl.w), qs, k, v, K - 1, K, rp, ci, q_index=idx, out=two, out_at_index=True)
    api.var_scatter_restore(base, hi, wi, None, idx, ho, wo, out=two)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    ib = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    got = out.view(ib).cpu().numpy().reshape(Bq * Hq, n, D)
    assert np.array_equal(got, two.view(ib).cpu().numpy().reshape(Bq * Hq, n, D)), "one launch vs two calls"
    upd = api.var_attn_block_sparse((wl.h, wl.w), qs, k, v, K - 1, K, rp, ci, q_index=idx, out_dtype=out_dtype)
    ref = oracle.scatter_restore(base.view(ib).cpu().numpy().reshape(Bq * Hq, -1, D), hi, wi,
                                 upd.view(ib).cpu().numpy().reshape(Bq * Hq, sel.size, D), sel, ho, wo)
    assert np.array_equal(got, ref), "oracle reconstruction"
    kept = oracle.tile_mask(wl.h, wl.w, K - 1, K, 64, 64, 7 if wl_name.startswith("var1024") else 3,
                            7 if wl_name.startswith("var1024") else 3, 2, 2, q_index=sel)
    qn, kn, vn = _np(qs), _np(k), _np(v)
    rows = np.arange(0, sel.size, 7)
    for (b, h) in ((0, 0), (Bq - 1, Hq - 1)):
        att = oracle.attention(qn[b:b + 1, h:h + 1], kn[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1], wl.h, wl.w,
                               K - 1, K, q_index=sel, kept=kept, rows=rows)
        _check(_np(out[b:b + 1, h:h + 1])[:, :, sel[rows]], att, what=f"restore {wl_name} {frac} b{b} h{h}")


def test_sparse_restore_edge_cases_and_errors(api):
    """No retained row: the launch is the upsampling alone.  Bad indices set the flag
    with every access in bounds.  Inputs outside the call's contract are refused
    before anything runs."""
    wl, q, k, v, K, n, sel, idx, qs, rp, ci, base = _restore_case(api, "var256", 2, 0.4)
    hi, wi, ho, wo = wl.h[-2], wl.w[-2], wl.h[-1], wl.w[-1]
    empty = torch.zeros(0, dtype=torch.int32, device="cuda")
    out = torch.full((2, 16, n, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    api.var_attn_block_sparse_restore((wl.h, wl.w), qs, k, v, K - 1, rp, ci, empty, base, hi, wi, out=out)
    ref = oracle.scatter_restore(base.view(torch.int16).cpu().numpy().reshape(32, -1, 64), hi, wi,
                                 np.zeros((32, 0, 64), np.int16), np.zeros(0, np.int32), ho, wo)
    assert np.array_equal(out.view(torch.int16).cpu().numpy().reshape(32, n, 64), ref)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    bad = torch.tensor([3, 3, 9], dtype=torch.int32, device="cuda")
    rpb, cib = api.var_build_tile_mask((wl.h, wl.w), K - 1, K, api.mask_params(64, 64, 3, 3, 2, 2), q_index=bad)
    api.var_attn_block_sparse_restore((wl.h, wl.w), qs, k, v, K - 1, rpb, cib, bad, base, hi, wi, out=out,
                                      err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) & 2
    VarAttnError = api.VarAttnError
    with pytest.raises(VarAttnError):   # fp32 input
        api.var_attn_block_sparse_restore((wl.h, wl.w), qs.float(), k.float(), v.float(), K - 1, rp, ci, idx,
                                          base.float(), hi, wi, out=out.float())
    with pytest.raises(ValueError):     # base of another dtype
        api.var_attn_block_sparse_restore((wl.h, wl.w), qs, k, v, K - 1, rp, ci, idx, base.float(), hi, wi,
                                          out=out)
    with pytest.raises(VarAttnError):   # rows of base not 16-byte aligned
        wide = torch.zeros(2, 16, hi * wi, 68, dtype=torch.bfloat16, device="cuda")
        api.var_attn_block_sparse_restore((wl.h, wl.w), qs, k, v, K - 1, rp, ci, idx, wide[..., :64], hi, wi,
                                          out=out)
