"""GPU parity of the key-split launches (var_attn_dense_split, var_attn_block_sparse_split).

A split changes only the order of the floating-point sums, so the bars are
those of the unsplit kernels: bf16 inputs max-abs <= 1e-2 and mean-abs <=
1e-3 against the fp64 oracle, LSE within lse_bound(L) (tests/_bounds.py; the
bf16 kernel's row sums add the bf16-rounded weights; each part's row sum is
within that factor of its exact value, and so is the merged sum), and two
kernel results within twice that of each other.
"""

import numpy as np
import pytest
import torch

import oracle
from _bounds import lse_bound
from scale_wise_attention_amd.inputs import WORKLOADS, make_qkv, pruned_index

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from scale_wise_attention_amd import api as _api
    return _api


def _np(t):
    return t.detach().float().cpu().numpy()


def _check(got, ref, what):
    err = np.abs(got.astype(np.float64) - ref)
    print(f"[{what}] max-abs {err.max():.3e} mean-abs {err.mean():.3e}", flush=True)
    assert err.max() <= 1e-2 and err.mean() <= 1e-3, what


def _ws(api, splits, q, rows):
    B, H, _, D = q.shape
    return api.split_workspace(splits, B, H, rows, D)


@pytest.mark.parametrize("step,splits", [(11, 2), (11, 3), (9, 2), (8, 8), (6, 3), (0, 8), (12, 2)])
def test_dense_split_steps_match_oracle(api, step, splits):
    wl = WORKLOADS["var1024"]
    q, k, v = make_qkv(wl, 3, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    qs = q[:, :, off[step]:off[step + 1]]
    n = off[step + 1] - off[step]
    o, lse = api.var_attn_dense((wl.h, wl.w), qs, k, v, step, step + 1, return_lse=True, n_splits=splits,
                                workspace=_ws(api, splits, q, n))
    rows = np.unique(np.concatenate([np.arange(0, n, max(1, n // 61)), [n - 1]]))
    qn, kn, vn = _np(qs), _np(k), _np(v)
    # (1, 12) and (1, 15): at step 11 (288 work items) the items past the
    # device's first round run split, the earlier ones whole
    for (b, h) in [(0, 0), (1, 9), (1, 12), (1, 15)]:
        ref, ref_lse = oracle.attention(qn[b:b + 1, h:h + 1], kn[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1],
                                        wl.h, wl.w, step, step + 1, rows=rows, return_lse=True)
        _check(_np(o[b:b + 1, h:h + 1])[:, :, rows], ref, f"dense step {step} x{splits} b{b} h{h}")
        assert np.max(np.abs(_np(lse[b:b + 1, h:h + 1])[:, :, rows] - ref_lse)) <= lse_bound(off[step + 1])


def test_dense_split_bf16_output_matches_unsplit(api):
    wl = WORKLOADS["var1024"]
    q, k, v = make_qkv(wl, 4, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    s = 11
    qs = q[:, :, off[s]:off[s + 1]]
    base = api.var_attn_dense((wl.h, wl.w), qs, k, v, s, s + 1, out_dtype=torch.bfloat16).float()
    ws = _ws(api, 3, q, off[s + 1] - off[s])
    for _ in range(2):        # the workspace is reused by a second call
        got = api.var_attn_dense((wl.h, wl.w), qs, k, v, s, s + 1, out_dtype=torch.bfloat16, n_splits=3,
                                 workspace=ws).float()
        d = (got - base).abs()
        print(f"[split vs unsplit] max {float(d.max()):.3e} mean {float(d.mean()):.3e}", flush=True)
        assert float(d.max()) <= 1e-2 and float(d.mean()) <= 1e-3


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dense_whole_and_split_items(api, out_dtype):
    """The 48x48 step: 9 query tiles x 32 (batch, head) = 288 work items, more
    than one round of a 256-CU device.  The items of the whole rounds run
    unsplit and write O directly; the rest run as 8 key splits and are merged.
    The workspace starts as NaN, so a merge over a whole item's rows, or a
    whole item's partial read back, shows as NaN.  Every row is compared with
    the unsplit launch, and rows of every (batch, head) with the oracle."""
    wl = WORKLOADS["var1024"]
    q, k, v = make_qkv(wl, 8, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    s = 11
    n = off[s + 1] - off[s]
    qs = q[:, :, off[s]:off[s + 1]]
    base, base_lse = api.var_attn_dense((wl.h, wl.w), qs, k, v, s, s + 1, out_dtype=out_dtype, return_lse=True)
    ws = _ws(api, 8, q, n).fill_(float("nan"))
    for rep in range(2):      # a second call over the first one's workspace
        o, lse = api.var_attn_dense((wl.h, wl.w), qs, k, v, s, s + 1, out_dtype=out_dtype, return_lse=True,
                                    n_splits=8, workspace=ws)
        assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
        d = (o.float() - base.float()).abs()
        print(f"[whole+split vs unsplit {out_dtype} call {rep}] max {float(d.max()):.3e} "
              f"mean {float(d.mean()):.3e}", flush=True)
        assert float(d.max()) <= 1e-2 and float(d.mean()) <= 1e-3
        assert float((lse - base_lse).abs().max()) <= 2 * lse_bound(off[s + 1])
    rows = np.unique(np.concatenate([np.arange(3, n, 97), [n - 1]]))
    qn, kn, vn = _np(qs), _np(k), _np(v)
    ref, ref_lse = oracle.attention(qn, kn, vn, wl.h, wl.w, s, s + 1, rows=rows, return_lse=True)
    _check(_np(o)[:, :, rows], ref, f"whole+split x8 {out_dtype}")
    assert np.max(np.abs(_np(lse)[:, :, rows] - ref_lse)) <= lse_bound(off[s + 1])


def test_full_sequence_split_rows_with_empty_parts(api):
    """Full-sequence mode: early rows see few keys, so several of their parts are empty."""
    wl = WORKLOADS["var256"]
    q, k, v = make_qkv(wl, 5, device="cuda")
    L = wl.tokens
    o, lse = api.var_attn_dense((wl.h, wl.w), q, k, v, 0, wl.num_scales, return_lse=True, n_splits=8,
                                workspace=_ws(api, 8, q, L))
    ref, ref_lse = oracle.attention(_np(q), _np(k), _np(v), wl.h, wl.w, 0, wl.num_scales, return_lse=True)
    _check(_np(o), ref, "var256 full sequence x8")
    assert np.max(np.abs(_np(lse) - ref_lse)) <= lse_bound(L)


def test_gathered_rows_split(api):
    wl = WORKLOADS["var1024"]
    q, k, v = make_qkv(wl, 6, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    s = 12
    sel = pruned_index(4096, 0.4, 2)
    idx = torch.from_numpy(sel).cuda()
    qs = q[:, :, off[s]:]
    o = api.var_attn_dense((wl.h, wl.w), qs, k, v, s, s + 1, q_index=idx, n_splits=4,
                           workspace=_ws(api, 4, q, sel.size))
    rows = np.arange(0, sel.size, 41)
    ref = oracle.attention(_np(qs)[:1, 3:4], _np(k)[:1, 3:4], _np(v)[:1, 3:4], wl.h, wl.w, s, s + 1,
                           q_index=sel, rows=rows)
    _check(_np(o[:1, 3:4])[:, :, rows], ref, "gathered x4")


@pytest.mark.parametrize("step,splits,pruned", [(11, 2, False), (10, 3, False), (12, 2, True), (8, 5, False)])
def test_sparse_split_matches_oracle(api, step, splits, pruned):
    wl = WORKLOADS["var1024_sparse"]
    q, k, v = make_qkv(wl, 7, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    qs = q[:, :, off[step]:off[step + 1]]
    sel = pruned_index(4096, 0.4, 0) if pruned else None
    idx = torch.from_numpy(sel).cuda() if pruned else None
    mp = api.mask_params()
    rp, ci = api.var_build_tile_mask((wl.h, wl.w), step, step + 1, mp, q_index=idx)
    n = sel.size if pruned else off[step + 1] - off[step]
    o, lse = api.var_attn_block_sparse((wl.h, wl.w), qs, k, v, step, step + 1, rp, ci, q_index=idx,
                                       return_lse=True, n_splits=splits, workspace=_ws(api, splits, q, n))
    kept = oracle.tile_mask(wl.h, wl.w, step, step + 1, 64, 64, 7, 7, 2, 2, q_index=sel)
    rows = np.unique(np.concatenate([np.arange(0, n, max(1, n // 53)), [n - 1]]))
    qn, kn, vn = _np(qs), _np(k), _np(v)
    for (b, h) in [(0, 2), (1, 14)]:
        ref, ref_lse = oracle.attention(qn[b:b + 1, h:h + 1], kn[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1],
                                        wl.h, wl.w, step, step + 1, q_index=sel, kept=kept, rows=rows,
                                        return_lse=True)
        _check(_np(o[b:b + 1, h:h + 1])[:, :, rows], ref, f"sparse step {step} x{splits} b{b} h{h}")
        assert np.max(np.abs(_np(lse[b:b + 1, h:h + 1])[:, :, rows] - ref_lse)) <= lse_bound(off[step + 1])


def test_split_plan_and_errors(api):
    wl = WORKLOADS["var1024"]
    n, nbytes = api.var_attn_split_plan((wl.h, wl.w), 11, 12, 2, 16, 128)
    # (256 compute units: items 256..287 split, 8192 rows from (b, h) 28, row 1024 on)
    assert 1 <= n <= 8 and nbytes == (n * 8192 * 129 * 4 if n > 1 else 0)
    q, k, v = make_qkv(wl, 0, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    # (the 24x24 step: 160 work items of 128 rows, fewer than the compute units,
    # so every item runs split and all 32 x 576 rows are partial rows; the
    # workspace holds 500 per map)
    qs = q[:, :, off[8]:off[9]]
    short = api.split_workspace(2, 2, 16, 500, 128)
    with pytest.raises(api.VarAttnError) as e:
        api.var_attn_dense((wl.h, wl.w), qs, k, v, 8, 9, n_splits=2, workspace=short)
    assert e.value.status_name == "VAR_ERR_CAPACITY"
    with pytest.raises(api.VarAttnError) as e:
        api.var_attn_dense((wl.h, wl.w), qs, k, v, 8, 9, n_splits=9, workspace=short)
    assert e.value.status_name == "VAR_ERR_RANGE"


def test_device_info_matches_torch(api):
    """The compute units the split plan assumes are the device's (torch reads them
    through its own HIP runtime), and the peak clock is a plausible engine clock."""
    cus, khz = api.var_device_info()
    assert cus == torch.cuda.get_device_properties(0).multi_processor_count
    assert 500_000 <= khz <= 5_000_000
