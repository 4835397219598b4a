"""The allocation-free key-split entry point (var_attn_dense_split_noalloc, through the
C ABI): its output equals var_attn_dense_split's with a caller workspace, bit for bit (the
same kernels, split plan and partial layout; only the partials' memory differs), on two
calls in a row, the second with a smaller input that reuses the scratch the first left
behind; and it matches the fp64 oracle at the bf16 bars."""

import numpy as np
import pytest
import torch

import oracle
from scale_wise_attention_amd.inputs import WORKLOADS, make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from scale_wise_attention_amd import api as _api
    return _api


def _call_pair(api, wl, q, k, v, s, n_splits, idx=None):
    off = oracle.offsets(wl.h, wl.w)
    qs = q[:, :, off[s]:off[s + 1]]
    B, H, D = q.shape[0], q.shape[1], q.shape[3]
    rows = off[s + 1] - off[s] if idx is None else idx.numel()
    ws = api.split_workspace(n_splits, B, H, rows, D)
    a = api.var_attn_dense(wl_sched(wl), qs, k, v, s, s + 1, q_index=idx, out_dtype=torch.bfloat16,
                           n_splits=n_splits, workspace=ws, return_lse=True)
    b = api.var_attn_dense_split_noalloc(wl_sched(wl), qs, k, v, s, s + 1, n_splits, q_index=idx,
                                         out_dtype=torch.bfloat16, return_lse=True)
    return a, b, qs


def wl_sched(wl):
    return (wl.h, wl.w)


def test_noalloc_matches_workspace_call_twice_second_smaller(api):
    wl = WORKLOADS["var1024"]
    q, k, v = make_qkv(wl, 21, device="cuda")
    # first: the 24x24 step, every work item (160 of 128 rows) split in 3 (28.5 MB
    # of partials); second: the 20x20 step split in 2 (fewer rows, 13.2 MB,
    # reusing what the first left)
    for s, n_splits in ((8, 3), (7, 2)):
        (oa, la), (ob, lb), qs = _call_pair(api, wl, q, k, v, s, n_splits)
        torch.cuda.synchronize()
        print(f"[noalloc step {s} x{n_splits}] equal: {torch.equal(oa, ob)} {torch.equal(la, lb)}", flush=True)
        assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)) and torch.equal(la, lb)
        ref = oracle.attention(qs[:1, :2].float().cpu().numpy(), k[:1, :2].float().cpu().numpy(),
                               v[:1, :2].float().cpu().numpy(), wl.h, wl.w, s, s + 1)
        err = np.abs(ob[:1, :2].float().cpu().numpy() - ref)
        assert err.max() <= 1e-2 and err.mean() <= 1e-3
    # a gathered call, and the 48x48 step (whole and split items in one launch)
    sel = torch.from_numpy(np.sort(np.random.default_rng(22).choice(2304, 1500, replace=False)).astype(np.int32)).cuda()
    for s, n_splits, idx in ((11, 6, None), (11, 2, sel)):   # (25 MB and 50 MB of partials)
        (oa, la), (ob, lb), _ = _call_pair(api, wl, q, k, v, s, n_splits, idx)
        assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)) and torch.equal(la, lb)


def test_noalloc_rejects_calls_beyond_the_scratch(api):
    wl = WORKLOADS["var1024"]
    q, k, v = make_qkv(wl, 23, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    # the 24x24 step split 8 ways needs 8 x 18432 x 129 x 4 bytes = 76 MB > 64 MiB
    with pytest.raises(api.VarAttnError) as e:
        api.var_attn_dense_split_noalloc(wl_sched(wl), q[:, :, off[8]:off[9]], k, v, 8, 9, 8)
    assert e.value.status_name == "VAR_ERR_CAPACITY"
