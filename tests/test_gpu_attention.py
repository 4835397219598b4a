"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Tolerances: float32 inputs max-abs <= 1e-5; bf16 inputs with float32
accumulation max-abs <= 1e-2 and mean-abs <= 1e-3 (both for fp32 and bf16
outputs); LSE within the bound the bf16 arithmetic gives (tests/_bounds.py);
tile masks, indices and scatter results bit-exact.
"""

import numpy as np
import pytest
import torch

import oracle
from _bounds import lse_bound
from _oracle_heads import attention_all_heads
from scale_wise_attention_amd.inputs import WORKLOADS, make_qkv, pruned_index

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5
BF16_MAX, BF16_MEAN = 1e-2, 1e-3


@pytest.fixture(scope="module")
def api():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from scale_wise_attention_amd import api as _api
    return _api


def _np(t):
    return t.detach().float().cpu().numpy()


def _sched(wl):
    return (wl.h, wl.w)


def _check(got, ref, dtype, what):
    err = np.abs(got.astype(np.float64) - ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    print(f"[{what}] max-abs {mx:.3e} mean-abs {mean:.3e}", flush=True)
    if dtype == "f32":
        assert mx <= F32_TOL, what
    else:
        assert mx <= BF16_MAX and mean <= BF16_MEAN, what


def _steps(api, wl, q, k, v, out_dtype=None):
    off = oracle.offsets(wl.h, wl.w)
    outs = []
    for s in range(wl.num_scales):
        qs = q[:, :, off[s]:off[s + 1]]
        outs.append(api.var_attn_dense(_sched(wl), qs, k, v, s, s + 1, out_dtype=out_dtype))
    return outs


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_fp32_steps_and_full_sequence(api, seed):
    wl = WORKLOADS["tiny_fp32"]
    q, k, v = make_qkv(wl, seed, device="cuda")
    qn, kn, vn = _np(q), _np(k), _np(v)
    off = oracle.offsets(wl.h, wl.w)
    for s, o in enumerate(_steps(api, wl, q, k, v)):
        ref = oracle.attention(qn[:, :, off[s]:off[s + 1]], kn, vn, wl.h, wl.w, s, s + 1)
        _check(_np(o), ref, "f32", f"tiny step {s}")
    o, lse = api.var_attn_dense(_sched(wl), q, k, v, 0, wl.num_scales, return_lse=True)
    ref, ref_lse = oracle.attention(qn, kn, vn, wl.h, wl.w, 0, wl.num_scales, return_lse=True)
    _check(_np(o), ref, "f32", "tiny full sequence")
    assert np.max(np.abs(_np(lse) - ref_lse)) <= F32_TOL
    # the first token sees only itself: O = v_0 exactly
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0].cpu())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_var256_all_steps_bf16(api, seed):
    wl = WORKLOADS["var256"]
    q, k, v = make_qkv(wl, seed, device="cuda")
    qn, kn, vn = _np(q), _np(k), _np(v)
    off = oracle.offsets(wl.h, wl.w)
    for s, o in enumerate(_steps(api, wl, q, k, v)):
        ref = oracle.attention(qn[:, :, off[s]:off[s + 1]], kn, vn, wl.h, wl.w, s, s + 1)
        _check(_np(o), ref, "bf16", f"var256 seed {seed} step {s}")


def test_var256_full_sequence_block_causal_and_lse(api):
    wl = WORKLOADS["var256"]
    q, k, v = make_qkv(wl, 5, device="cuda")
    o, lse = api.var_attn_dense(_sched(wl), q, k, v, 0, wl.num_scales, return_lse=True)
    ref, ref_lse = oracle.attention(_np(q), _np(k), _np(v), wl.h, wl.w, 0, wl.num_scales, return_lse=True)
    _check(_np(o), ref, "bf16", "var256 full sequence")
    lerr = float(np.max(np.abs(_np(lse) - ref_lse)))
    print(f"[var256 full sequence] lse max-abs {lerr:.3e} (bound {lse_bound(680):.3e})", flush=True)
    assert lerr <= lse_bound(680)
    # scale-1 query: its only key is token 0, so O = v_0 exactly.  Its one weight is
    # exp2 of the rounding error of the fused scale-and-shift, within 2^-20 of 1, which
    # rounds to 1.0 in bf16: the PV product and the row sum both see exactly 1.
    assert torch.equal(o[:, :, 0], v[:, :, 0].float())
    ob = api.var_attn_dense(_sched(wl), q, k, v, 0, wl.num_scales, out_dtype=torch.bfloat16)
    assert torch.equal(ob[:, :, 0].view(torch.int16), v[:, :, 0].view(torch.int16))
    # the same in step mode (the 1x1 step alone), fp32 and bf16 output
    for odt in (torch.float32, torch.bfloat16):
        o0 = api.var_attn_dense(_sched(wl), q[:, :, :1], k, v, 0, 1, out_dtype=odt)
        assert torch.equal(o0[:, :, 0].float(), v[:, :, 0].float())
    # a middle range of scales
    off = oracle.offsets(wl.h, wl.w)
    o2 = api.var_attn_dense(_sched(wl), q[:, :, off[3]:off[7]], k, v, 3, 7)
    ref2 = oracle.attention(_np(q)[:, :, off[3]:off[7]], _np(k), _np(v), wl.h, wl.w, 3, 7)
    _check(_np(o2), ref2, "bf16", "var256 scales 3..6")


def test_var256_bf16_output(api):
    wl = WORKLOADS["var256"]
    q, k, v = make_qkv(wl, 3, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    s = wl.num_scales - 1
    o = api.var_attn_dense(_sched(wl), q[:, :, off[s]:], k, v, s, s + 1, out_dtype=torch.bfloat16)
    assert o.dtype == torch.bfloat16
    ref = oracle.attention(_np(q)[:, :, off[s]:], _np(k), _np(v), wl.h, wl.w, s, s + 1)
    _check(_np(o), ref, "bf16", "var256 last step bf16 out")


def test_var512_all_steps(api):
    wl = WORKLOADS["var512"]
    q, k, v = make_qkv(wl, 0, device="cuda")
    qn, kn, vn = _np(q), _np(k), _np(v)
    off = oracle.offsets(wl.h, wl.w)
    for s, o in enumerate(_steps(api, wl, q, k, v)):
        ref = oracle.attention(qn[:, :, off[s]:off[s + 1]], kn, vn, wl.h, wl.w, s, s + 1)
        _check(_np(o), ref, "bf16", f"var512 step {s}")


def test_gather_rows_match_oracle_and_dense_rows(api):
    wl = WORKLOADS["var512"]
    q, k, v = make_qkv(wl, 1, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    s = wl.num_scales - 1
    qs = q[:, :, off[s]:]
    n_q = off[s + 1] - off[s]
    for sel in (pruned_index(n_q, 0.4, 1), np.array([n_q - 1], np.int32), np.arange(n_q, dtype=np.int32)[::-7].copy()):
        idx = torch.from_numpy(sel).cuda()
        o = api.var_attn_dense(_sched(wl), qs, k, v, s, s + 1, q_index=idx)
        ref = oracle.attention(_np(qs), _np(k), _np(v), wl.h, wl.w, s, s + 1, q_index=sel)
        _check(_np(o), ref, "bf16", f"var512 gather n_sel={sel.size}")
        full = api.var_attn_dense(_sched(wl), qs, k, v, s, s + 1)
        # the same query computed in another tile: equal up to the bf16 rounding of its weights
        assert float((o - full[:, :, idx.long()]).abs().max()) <= 5e-3


def test_empty_selection_is_a_noop(api):
    wl = WORKLOADS["var256"]
    q, k, v = make_qkv(wl, 0, device="cuda")
    idx = torch.zeros(0, dtype=torch.int32, device="cuda")
    o = api.var_attn_dense(_sched(wl), q[:, :, 424:], k, v, 9, 10, q_index=idx)
    assert o.shape == (2, 16, 0, 64)
    rp, ci = api.var_build_tile_mask(_sched(wl), 9, 10, api.mask_params(), q_index=idx)
    assert rp.cpu().tolist() == [0]
    o = api.var_attn_block_sparse(_sched(wl), q[:, :, 424:], k, v, 9, 10, rp, ci, q_index=idx)
    assert o.shape == (2, 16, 0, 64)


def test_var1024_last_step_full_size(api):
    """Full 1024px last step (4096 x 10521, B=2, H=16, D=128) as the benchmark launches it
    (bf16 output, grid 512 x 256): every (batch, head) and every row against the oracle."""
    wl = WORKLOADS["var1024"]
    q, k, v = make_qkv(wl, 0, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    s = wl.num_scales - 1
    qs = q[:, :, off[s]:]
    o, lse = api.var_attn_dense(_sched(wl), qs, k, v, s, s + 1, out_dtype=torch.bfloat16, return_lse=True)
    ref, ref_lse = attention_all_heads(_np(qs), _np(k), _np(v), wl.h, wl.w, s, s + 1, return_lse=True)
    _check(_np(o), ref, "bf16", "var1024 last step, all 32 (b, h), all rows")
    lerr = float(np.max(np.abs(_np(lse) - ref_lse)))
    print(f"[var1024 last step] lse max-abs {lerr:.3e} (bound {lse_bound(10521):.3e})", flush=True)
    assert lerr <= lse_bound(10521)


def test_var1024_generation_steps_as_benchmarked(api):
    """Steps 1..12 of the 1024px generation in the benchmark's launch configuration (the
    library's split plan per step, bf16 output): every (batch, head) and every row."""
    wl = WORKLOADS["var1024"]
    q, k, v = make_qkv(wl, 1, device="cuda")
    qn, kn, vn = _np(q), _np(k), _np(v)
    off = oracle.offsets(wl.h, wl.w)
    B, H, D = wl.batch, wl.heads, wl.head_dim
    for s in range(wl.num_scales - 1):
        n_splits, ws_bytes = api.var_attn_split_plan(_sched(wl), s, s + 1, B, H, D)
        ws = torch.empty(max(1, ws_bytes // 4), dtype=torch.float32, device="cuda").fill_(float("nan"))
        o = api.var_attn_dense(_sched(wl), q[:, :, off[s]:off[s + 1]], k, v, s, s + 1, out_dtype=torch.bfloat16,
                               n_splits=n_splits, workspace=ws)
        ref = attention_all_heads(qn[:, :, off[s]:off[s + 1]], kn, vn, wl.h, wl.w, s, s + 1)
        _check(_np(o), ref, "bf16", f"var1024 step {s} ({n_splits} key splits), all (b, h), all rows")


def test_deterministic_runs(api):
    wl = WORKLOADS["var512"]
    q, k, v = make_qkv(wl, 2, device="cuda")
    a = api.var_attn_dense(_sched(wl), q[:, :, 1216:], k, v, 9, 10)
    b = api.var_attn_dense(_sched(wl), q[:, :, 1216:], k, v, 9, 10)
    assert torch.equal(a, b)


def test_strided_views(api):
    """Non-contiguous [B, H, T, D] views (token-major storage) go through the strides."""
    wl = WORKLOADS["var256"]
    q, k, v = make_qkv(wl, 4, device="cuda")
    qt = q.transpose(1, 2).contiguous().transpose(1, 2)   # storage [B, T, H, D]
    kt = k.transpose(1, 2).contiguous().transpose(1, 2)
    vt = v.transpose(1, 2).contiguous().transpose(1, 2)
    s = wl.num_scales - 1
    a = api.var_attn_dense(_sched(wl), q[:, :, 424:], k, v, s, s + 1)
    b = api.var_attn_dense(_sched(wl), qt[:, :, 424:], kt, vt, s, s + 1)
    assert torch.equal(a, b)


def test_invalid_shapes_raise_before_launch(api):
    wl = WORKLOADS["var256"]
    q, k, v = make_qkv(wl, 0, device="cuda")
    with pytest.raises(ValueError):
        api.var_attn_dense(_sched(wl), q[:, :, :10], k, v, 9, 10)          # too few query rows
    with pytest.raises(ValueError):
        api.var_attn_dense(_sched(wl), q, k[:, :, :100], v, 9, 10)         # KV shorter than kv_len
    with pytest.raises(api.VarAttnError):
        api.var_attn_dense(_sched(wl), q, k, v, 9, 11)                     # bad scale range


def test_branch_halving_cond_only_call_equals_cond_half(api):
    """Branch Halving ("ARVAR ...", Key Design 1) at the attention level: the
    step runs the conditional branch alone (a batch-1 call on batch entry 0)
    and its output stands for both branches.  The batch-1 call is checked
    against the oracle on the conditional branch (every head and row of the
    1024px last step), and, since each (batch, head) is computed
    independently, against the conditional half of the two-branch call bit
    for bit, dense and block-sparse."""
    wl = WORKLOADS["var1024_sparse"]
    q, k, v = make_qkv(wl, 1, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    K = wl.num_scales
    qs = q[:, :, off[K - 1]:]
    cond = api.var_attn_dense(_sched(wl), qs[:1], k[:1], v[:1], K - 1, K, out_dtype=torch.bfloat16)
    ref = attention_all_heads(_np(qs[:1]), _np(k[:1]), _np(v[:1]), wl.h, wl.w, K - 1, K)
    _check(_np(cond), ref, "bf16", "branch halving: cond-only last step vs oracle")
    repeated = cond.expand(2, -1, -1, -1)          # the repeat that restores the two-branch interface
    for b in range(2):
        _check(_np(repeated[b:b + 1]), ref, "bf16", f"branch halving: repeated output, branch {b}")
    both = api.var_attn_dense(_sched(wl), qs, k, v, K - 1, K, out_dtype=torch.bfloat16)
    assert torch.equal(cond.view(torch.int16), both[:1].view(torch.int16))
    assert torch.equal(repeated[1].view(torch.int16), both[0].view(torch.int16))
    mp = api.mask_params()
    rp, ci = api.var_build_tile_mask(_sched(wl), K - 1, K, mp)
    both_s = api.var_attn_block_sparse(_sched(wl), qs, k, v, K - 1, K, rp, ci)
    cond_s = api.var_attn_block_sparse(_sched(wl), qs[:1], k[:1], v[:1], K - 1, K, rp, ci)
    assert torch.equal(cond_s, both_s[:1])
