"""GPU parity of the attention-guided selection: saliency and Top-K.

Saliency is compared with the float64 oracle.  Given the oracle's own LSE the
only error left is fp32 arithmetic (MFMA accumulation of exact bf16 products,
v_exp_f32), bounded here by 1e-4 relative.  Given the LSE of the bf16
attention kernel (whose row sums add the bf16-rounded weights: within
lse_bound(L) of the exact LSE, tests/_bounds.py), every weight, and so every
saliency (a sum of positive weights), is within exp(lse_bound(L)) - 1 + 1e-4
relative.  The Top-K choice is an
integer result: the oracle applied to the same float32 maps must give the
same positions bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
from _bounds import lse_bound
from scale_wise_attention_amd.inputs import WORKLOADS, make_qkv, custom_workload, pruned_index

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from scale_wise_attention_amd import api as _api
    return _api


def _rel(got, ref, what):
    err = np.abs(got.astype(np.float64) - ref) / np.abs(ref)
    print(f"[{what}] max rel {err.max():.3e} mean rel {err.mean():.3e}", flush=True)
    return err.max()


def _saliency_case(api, wl, step, seed, heads=None):
    q, k, v = make_qkv(wl, seed, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    qs = q[:, :, off[step]:off[step + 1]]
    kn, vn, qn = k.float().cpu().numpy(), v.float().cpu().numpy(), qs.float().cpu().numpy()
    ref = oracle.saliency(qn, kn, wl.h, wl.w, step)
    _, ref_lse = oracle.attention(qn, kn, vn, wl.h, wl.w, step, step + 1, return_lse=True)
    lse_exact = torch.from_numpy(ref_lse.astype(np.float32)).cuda()
    got_exact = api.var_attn_saliency((wl.h, wl.w), qs, k, lse_exact, step).cpu().numpy()
    _, lse_gpu = api.var_attn_dense((wl.h, wl.w), qs, k, v, step, step + 1, return_lse=True)
    got_gpu = api.var_attn_saliency((wl.h, wl.w), qs, k, lse_gpu, step).cpu().numpy()
    return got_exact, got_gpu, ref


@pytest.mark.parametrize("wl_name,step", [("var1024", 9), ("var1024", 6), ("var256", 7), ("var256", 2),
                                          ("var512", 8)])
def test_saliency_matches_oracle(api, wl_name, step):
    wl = WORKLOADS[wl_name]
    got_exact, got_gpu, ref = _saliency_case(api, wl, step, 0)
    assert _rel(got_exact, ref, f"{wl_name} step {step}, oracle lse") <= 1e-4
    L = oracle.offsets(wl.h, wl.w)[step + 1]
    assert _rel(got_gpu, ref, f"{wl_name} step {step}, kernel lse") <= np.expm1(lse_bound(L)) + 1e-4


def test_saliency_single_token_scale_is_one(api):
    wl = WORKLOADS["var1024"]
    got_exact, got_gpu, ref = _saliency_case(api, wl, 0, 1)
    assert np.array_equal(ref, np.ones_like(ref))
    assert np.max(np.abs(got_exact - 1.0)) <= 1e-6


def _check_select(api, maps, hs, ws, hd, wd, n_keep, what):
    t = torch.from_numpy(np.ascontiguousarray(maps, dtype=np.float32)).cuda()
    got = api.var_select_topk(t, hs, ws, hd, wd, n_keep).cpu().numpy()
    ref = oracle.select_positions(maps, hs, ws, hd, wd, n_keep)
    print(f"[select {what}] n_keep {n_keep} first {got[:4].tolist()}", flush=True)
    assert got.dtype == np.int32 and np.array_equal(got, ref), what


def test_select_on_kernel_saliency_1024(api):
    """Saliency of the 32x32 step upsampled to 64x64, keep 40% (1638 positions)."""
    wl = WORKLOADS["var1024"]
    q, k, v = make_qkv(wl, 2, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    qs = q[:, :, off[9]:off[10]]
    _, lse = api.var_attn_dense((wl.h, wl.w), qs, k, v, 9, 10, return_lse=True)
    sal = api.var_attn_saliency((wl.h, wl.w), qs, k, lse, 9)
    maps = sal.cpu().numpy().reshape(-1, 1024)
    _check_select(api, maps, 32, 32, 64, 64, 1638, "1024 32->64")
    _check_select(api, maps, 32, 32, 64, 64, 1024, "1024 32->64 quarter")


@pytest.mark.parametrize("seed", range(12))
def test_select_random_maps_with_ties(api, seed):
    rng = np.random.default_rng(700 + seed)
    hs, ws = int(rng.integers(1, 40)), int(rng.integers(1, 40))
    hd, wd = hs + int(rng.integers(0, 40)), ws + int(rng.integers(0, 40))
    n_maps = int(rng.integers(1, 6))
    levels = int(rng.integers(1, 9))
    maps = (np.round(rng.random((n_maps, hs * ws)) * levels) / levels).astype(np.float32)
    if seed % 3 == 0:
        maps[:, ::5] = -0.0
    n_keep = int(rng.integers(1, hd * wd + 1))
    _check_select(api, maps, hs, ws, hd, wd, n_keep, f"random {seed}")


def test_select_edge_cases(api):
    flat = np.full((2, 12), 0.5, np.float32)
    _check_select(api, flat, 3, 4, 6, 8, 48, "keep all")
    _check_select(api, flat, 3, 4, 6, 8, 1, "keep one of equals")
    _check_select(api, flat, 3, 4, 3, 4, 5, "same grid")
    spread = np.linspace(-3, 3, 64 * 64, dtype=np.float32).reshape(1, -1)
    _check_select(api, spread, 64, 64, 64, 64, 4095, "negative scores")
    big = np.array([[2.0 ** 24, 2.0 ** 24], [1.0, 0.0], [1.0, 2.0]], np.float32)
    _check_select(api, big, 1, 2, 1, 2, 1, "float32 order")
    assert api.var_select_topk(torch.zeros(1, 4, device="cuda"), 2, 2, 4, 4, 0).numel() == 0
    rng = np.random.default_rng(5)
    coarse = (np.round(rng.random((3, 24 * 24)) * 16) / 16).astype(np.float32)
    _check_select(api, coarse, 24, 24, 96, 96, 3000, "destination above the LDS cache")
    _check_select(api, rng.random((32, 90 * 90)).astype(np.float32), 90, 90, 91, 90, 4000, "largest source")


def test_selection_drives_the_pruned_pipeline(api):
    """Saliency (32x32) -> Top-K on 64x64 -> tile mask + sparse attention + scatter."""
    wl = WORKLOADS["var1024_sparse"]
    q, k, v = make_qkv(wl, 0, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    K = wl.num_scales
    qs9 = q[:, :, off[9]:off[10]]
    _, lse = api.var_attn_dense((wl.h, wl.w), qs9, k, v, 9, 10, return_lse=True)
    sal = api.var_attn_saliency((wl.h, wl.w), qs9, k, lse, 9)
    idx = api.var_select_topk(sal, 32, 32, 64, 64, 1638)
    sel = idx.cpu().numpy()
    assert np.array_equal(sel, oracle.select_positions(sal.cpu().numpy().reshape(-1, 1024), 32, 32, 64, 64, 1638))
    mp = api.mask_params()
    rp, ci = api.var_build_tile_mask((wl.h, wl.w), K - 1, K, mp, q_index=idx)
    kept = oracle.tile_mask(wl.h, wl.w, K - 1, K, 64, 64, 7, 7, 2, 2, q_index=sel)
    erp, eci = oracle.mask_to_csr(kept)
    assert np.array_equal(rp.cpu().numpy(), erp) and np.array_equal(ci.cpu().numpy()[: erp[-1]], eci)
    upd = api.var_attn_block_sparse((wl.h, wl.w), q[:, :, off[K - 1]:], k, v, K - 1, K, rp, ci, q_index=idx)
    rows = np.arange(0, 1638, 97)
    qn, kn, vn = (t.float().cpu().numpy() for t in (q[:, :, off[K - 1]:], k, v))
    for (b, h) in ((0, 0), (1, 15)):
        ref = oracle.attention(qn[b:b + 1, h:h + 1], kn[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1], wl.h, wl.w,
                               K - 1, K, q_index=sel, kept=kept, rows=rows)
        err = np.abs(upd[b:b + 1, h:h + 1, rows].float().cpu().numpy() - ref)
        assert err.max() <= 1e-2 and err.mean() <= 1e-3
    base = api.var_attn_dense((wl.h, wl.w), q[:, :, off[K - 2]:off[K - 1]], k, v, K - 2, K - 1)
    out = api.var_scatter_restore(base, 48, 48, upd, idx, 64, 64)
    ref = oracle.scatter_restore(base.view(torch.int32).cpu().numpy(), 48, 48, upd.view(torch.int32).cpu().numpy(),
                                 sel, 64, 64)
    assert np.array_equal(out.view(torch.int32).cpu().numpy(), ref)


def test_selection_overlap_with_exact_saliency_1024(api):
    """How far the retained set moves when the kernel's saliency (float32, from the bf16
    attention kernel's LSE) drives the Top-K instead of the exact float64 saliency of the
    oracle (summed and ranked in float64): the fraction of the 1638 positions both keep.
    The integer choice itself is checked bit for bit on equal maps above; this measures the
    end-to-end effect of the float arithmetic on the 1024px shapes (32x32 -> 64x64)."""
    wl = WORKLOADS["var1024"]
    for seed in (0, 1, 2):
        q, k, v = make_qkv(wl, seed, device="cuda")
        off = oracle.offsets(wl.h, wl.w)
        qs = q[:, :, off[9]:off[10]]
        _, lse = api.var_attn_dense((wl.h, wl.w), qs, k, v, 9, 10, return_lse=True)
        sal = api.var_attn_saliency((wl.h, wl.w), qs, k, lse, 9)
        got = api.var_select_topk(sal, 32, 32, 64, 64, 1638).cpu().numpy()
        exact = oracle.saliency(qs.float().cpu().numpy(), k.float().cpu().numpy(), wl.h, wl.w, 9)
        score = exact.reshape(-1, 1024).sum(axis=0)[oracle.nearest_source_index(32, 32, 64, 64)]
        order = np.lexsort((np.arange(score.size), -score))
        ref = np.sort(order[:1638])
        overlap = np.intersect1d(got, ref).size / 1638
        print(f"[selection overlap, seed {seed}] {overlap:.4f} of 1638 positions kept by both", flush=True)
        assert overlap >= 0.95
