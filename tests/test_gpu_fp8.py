"""GPU parity of the e4m3 path: the quantiser bit for bit against the oracle's
quantize_tiles (codes and the scales of 64-token tiles), and attention with
e4m3 logits against the fp64 oracle on the dequantised values (keys
quantised per 64-token tile of the cache, queries per 64 output rows of the
call), at the bf16 bars (max-abs 1e-2, mean-abs 1e-3).  The LSE bar is
derived (tests/_bounds.py): the bf16 path's lse_bound(L) plus, per row, the
e4m3 matrix instruction's accumulation error, at most 2^-11.8 of the sum of
the product magnitudes (its documented worst case), times the softmax scale.
"""

import numpy as np
import pytest
import torch

import oracle
from _bounds import e4m3_logit_error, lse_bound
from _oracle_heads import attention_all_heads
from oracle.fp8 import dequantize_tiles, quantize_tiles
from scale_wise_attention_amd.inputs import WORKLOADS, custom_workload, make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from scale_wise_attention_amd import api as _api
    return _api


def _np(t):
    return t.detach().float().cpu().numpy()


def _oracle_quant(x):
    """x bf16 [B, H, T, D] (any device) -> oracle codes [B, H, T, D] and tile scales [B, H, ceil(T/64)]."""
    return quantize_tiles(_np(x))


def _check_quant(api, x, what):
    codes, scale = api.var_quantize_e4m3(x)
    ref_c, ref_s = _oracle_quant(x)
    got_c, got_s = codes.cpu().numpy(), scale.cpu().numpy()
    bad = np.count_nonzero(got_c != ref_c)
    print(f"[quant {what}] shape {tuple(x.shape)} code mismatches {bad}", flush=True)
    assert bad == 0
    assert np.array_equal(got_s.view(np.uint32), ref_s.view(np.uint32))
    return codes, scale, ref_c, ref_s


@pytest.mark.parametrize("D,T", [(128, 77), (64, 1), (16, 300), (128, 4096)])
def test_quantize_matches_oracle(api, D, T):
    rng = np.random.default_rng(40 + D + T)
    B, H = 2, 3
    x = rng.standard_normal((B, H, T, D)).astype(np.float32)
    x *= np.array([1.0, 1e-3, 40.0, 1.0, 0.0, 1.0], np.float32).reshape(B, H, 1, 1)
    x[1, 0, 0, 0] = 1e4          # one large value: the rest of the map falls into subnormal codes
    x[0, 0, :, 1] = -0.0         # negative zeros keep their sign bit
    _check_quant(api, torch.from_numpy(x).to(torch.bfloat16).cuda(), f"D={D}")


def test_quantize_ties_between_codes(api):
    # bf16 values placed so that x * 448 / amax lands on midpoints between e4m3 codes
    # (amax = 448 makes inv exactly 1): round half to even must pick the even code
    pos = np.array([1.0 + i / 8 for i in range(8)], np.float64)
    mids = np.concatenate([(pos[:-1] + pos[1:]) / 2 * 2.0 ** e for e in range(-6, 8)] +
                          [(pos[:6] + pos[1:7]) / 2 * 2.0 ** 8] +
                          [np.arange(1, 16) * 2.0 ** -10])   # subnormal codes and their midpoints
    x = np.zeros((1, 1, 1, 128), np.float32)
    flat = x.reshape(-1)
    flat[: mids.size] = mids
    flat[mids.size] = 448.0
    xt = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(xt.float().numpy().reshape(-1)[: mids.size], mids.astype(np.float32))  # exact in bf16
    _check_quant(api, xt.cuda(), "ties")


def test_quantize_strided_views_and_empty(api):
    wl = WORKLOADS["var1024"]
    q, k, _ = make_qkv(wl, 3, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    _check_quant(api, q[:, :, off[10]:off[11]], "q step view")
    big = torch.zeros((2, 2, 40, 256), dtype=torch.bfloat16, device="cuda")
    big[..., :128] = k[:, :2, :40]
    _check_quant(api, big[..., :128], "wide rows")
    codes, scale = api.var_quantize_e4m3(k[:, :, :0])
    assert codes.numel() == 0 and scale.numel() == 0


def test_quantize_var1024_full_cache_sampled_maps(api):
    """Full-size K cache (10521 tokens); the maps are independent, so a few are compared in full."""
    wl = WORKLOADS["var1024"]
    _, k, _ = make_qkv(wl, 5, device="cuda")
    codes, scale = api.var_quantize_e4m3(k)
    for b, h in [(0, 0), (0, 13), (1, 7), (1, 15)]:
        ref_c, ref_s = quantize_tiles(_np(k[b:b + 1, h:h + 1]))
        assert np.array_equal(codes[b, h].cpu().numpy(), ref_c[0, 0])
        assert np.array_equal(scale[b, h].cpu().numpy().view(np.uint32), ref_s[0, 0].view(np.uint32))


def test_quantize_growing_cache_touches_only_new_tiles(api):
    """Step by step over a schedule: each call requantises from the step's first token on."""
    wl = custom_workload(SMALL, 2, 2, 128)
    _, k, _ = make_qkv(wl, 6, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    codes = torch.full(k.shape, 0x55, dtype=torch.uint8, device="cuda")
    scale = torch.full((2, 2, -(-k.shape[2] // 64)), -1.0, dtype=torch.float32, device="cuda")
    for st in range(len(SMALL)):
        before_c, before_s = codes.clone(), scale.clone()
        api.var_quantize_e4m3(k[:, :, :off[st + 1]], codes=codes[:, :, :off[st + 1]], scale=scale,
                              first_token=off[st])
        t0 = off[st] // 64 * 64
        assert torch.equal(codes[:, :, :t0], before_c[:, :, :t0]) and torch.equal(codes[:, :, off[st + 1]:],
                                                                                   before_c[:, :, off[st + 1]:])
        assert torch.equal(scale[:, :, :t0 // 64], before_s[:, :, :t0 // 64])
        n_t = -(-off[st + 1] // 64)
        assert torch.equal(scale[:, :, n_t:], before_s[:, :, n_t:])
    ref_c, ref_s = _oracle_quant(k)
    assert np.array_equal(codes.cpu().numpy(), ref_c)
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


def _quantised(api, q, k, sel=None):
    """GPU codes of k (checked equal to the oracle's) with the oracle's dequantised keys, and the
    oracle's dequantised queries: the call's rows (q, or q[:, :, sel]) in groups of 64, placed back
    at their positions of q."""
    k8, sk, rk, rsk = _check_quant(api, k, "k")
    qn = _np(q)
    rows = qn if sel is None else qn[:, :, sel]
    qd_rows = dequantize_tiles(*quantize_tiles(rows))
    qd = np.zeros(qn.shape)
    if sel is None:
        qd = qd_rows
    else:
        qd[:, :, sel] = qd_rows
    return k8, sk, qd, dequantize_tiles(rk, rsk)


def _lse_bar(qd, kd, L, sel=None):
    """LSE bar of an e4m3 call whose rows see at most the L keys of kd: the bf16 path's bound
    plus the largest e4m3 logit error of any row (scale 1/sqrt(128))."""
    return lse_bound(L) + float(e4m3_logit_error(qd, np.asarray(kd)[:, :, :L], 128 ** -0.5, q_index=sel).max())


def _bars(got, ref, what, lse=None, ref_lse=None, lse_bar=None):
    err = np.abs(got.astype(np.float64) - ref)
    lerr = 0.0 if lse is None else float(np.max(np.abs(lse - ref_lse)))
    bar = f" (bar {lse_bar:.3e})" if lse_bar is not None else ""
    print(f"[{what}] max-abs {err.max():.3e} mean-abs {err.mean():.3e} lse {lerr:.3e}{bar}", flush=True)
    assert err.max() <= 1e-2 and err.mean() <= 1e-3
    if lse is not None:
        assert lerr <= lse_bar


SMALL = (1, 2, 4, 6, 8, 12, 16, 20)


@pytest.mark.parametrize("step", [0, 3, 5, 7])
def test_dense_e4m3_steps_match_oracle(api, step):
    wl = custom_workload(SMALL, 2, 2, 128, sink_offset_scales=3)
    q, k, v = make_qkv(wl, 60 + step, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    qs = q[:, :, off[step]:off[step + 1]].contiguous()
    kc = k[:, :, :off[step + 1]].contiguous()
    k8, sk, qd, kd = _quantised(api, qs, kc)
    o, lse = api.var_attn_dense_e4m3((wl.h, wl.w), qs, k8, sk, v, step, step + 1, return_lse=True)
    ref, ref_lse = oracle.attention(qd, kd, _np(v), wl.h, wl.w, step, step + 1, return_lse=True)
    _bars(_np(o), ref, f"e4m3 dense step {step}", _np(lse), ref_lse, _lse_bar(qd, kd, off[step + 1]))


def test_dense_e4m3_gather_splits_bf16_out(api):
    wl = custom_workload(SMALL, 2, 2, 128)
    q, k, v = make_qkv(wl, 70, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    s = 7
    qs = q[:, :, off[s]:off[s + 1]]
    n = off[s + 1] - off[s]
    sel = np.random.default_rng(71).choice(n, 157, replace=False).astype(np.int32)   # any order
    k8, sk, qd, kd = _quantised(api, qs, k, sel)
    idx = torch.from_numpy(sel).cuda()
    ref, ref_lse = oracle.attention(qd, kd, _np(v), wl.h, wl.w, s, s + 1, q_index=sel, return_lse=True)
    for splits in (1, 3):
        ws = api.split_workspace(splits, 2, 2, sel.size, 128) if splits > 1 else None
        for odt in (torch.float32, torch.bfloat16):
            o, lse = api.var_attn_dense_e4m3((wl.h, wl.w), qs, k8, sk, v, s, s + 1, q_index=idx, out_dtype=odt,
                                             return_lse=True, n_splits=splits, workspace=ws)
            _bars(_np(o), ref, f"e4m3 gather splits={splits} {odt}", _np(lse), ref_lse,
                  _lse_bar(qd, kd, off[s + 1], sel))


def test_dense_e4m3_tile_scales_differ(api):
    """Tiles of very different magnitude (scales 1/8 .. 8 apart), with and without key splits.

    Logits grow up to 16-fold, so most rows are dominated by one key; the LSE bar is the
    derived one, whose e4m3 term grows with the logits."""
    wl = custom_workload(SMALL, 2, 2, 128)
    q, k, v = make_qkv(wl, 77, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    s = 7
    rng = np.random.default_rng(78)
    kf = torch.from_numpy(np.repeat(2.0 ** rng.integers(-3, 4, -(-k.shape[2] // 64)), 64)[: k.shape[2]])
    k = (k.float() * kf.to("cuda", torch.float32)[None, None, :, None]).to(torch.bfloat16)
    n = off[s + 1] - off[s]
    qf = torch.from_numpy(np.repeat(2.0 ** rng.integers(-2, 2, -(-n // 64)), 64)[:n])
    qs = (q[:, :, off[s]:off[s + 1]].float() * qf.to("cuda", torch.float32)[None, None, :, None]).to(torch.bfloat16)
    k8, sk, qd, kd = _quantised(api, qs, k)
    ref, ref_lse = oracle.attention(qd, kd, _np(v), wl.h, wl.w, s, s + 1, return_lse=True)
    for splits in (1, 4):
        ws = api.split_workspace(splits, 2, 2, n, 128) if splits > 1 else None
        o, lse = api.var_attn_dense_e4m3((wl.h, wl.w), qs, k8, sk, v, s, s + 1, return_lse=True,
                                         n_splits=splits, workspace=ws)
        _bars(_np(o), ref, f"e4m3 tile scales differ splits={splits}", _np(lse), ref_lse,
              _lse_bar(qd, kd, off[s + 1]))


def test_dense_e4m3_multi_scale_call(api):
    """Queries of several scales in one call: each row sees keys up to the end of its own scale."""
    wl = custom_workload(SMALL, 1, 2, 128)
    q, k, v = make_qkv(wl, 72, device="cuda")
    k8, sk, qd, kd = _quantised(api, q, k)
    o, lse = api.var_attn_dense_e4m3((wl.h, wl.w), q, k8, sk, v, 0, len(SMALL), return_lse=True)
    ref, ref_lse = oracle.attention(qd, kd, _np(v), wl.h, wl.w, 0, len(SMALL), return_lse=True)
    _bars(_np(o), ref, "e4m3 all scales", _np(lse), ref_lse, _lse_bar(qd, kd, wl.tokens))


def test_dense_e4m3_var1024_last_step_full_size(api):
    """The e4m3 1024px last step as the benchmark launches it (bf16 output): every (batch, head)
    and row against the oracle on the oracle's own dequantised queries and keys."""
    wl = WORKLOADS["var1024"]
    q, k, v = make_qkv(wl, 73, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    s = len(wl.grids) - 1
    qs = q[:, :, off[s]:off[s + 1]]
    k8, sk = api.var_quantize_e4m3(k)
    o, lse = api.var_attn_dense_e4m3((wl.h, wl.w), qs, k8, sk, v, s, s + 1, return_lse=True,
                                     out_dtype=torch.bfloat16)
    rq, rsq = quantize_tiles(_np(qs))
    rk, rsk = quantize_tiles(_np(k))
    assert np.array_equal(k8.cpu().numpy(), rk)
    qd, kd = dequantize_tiles(rq, rsq), dequantize_tiles(rk, rsk)
    ref, ref_lse = attention_all_heads(qd, kd, _np(v), wl.h, wl.w, s, s + 1, return_lse=True)
    _bars(_np(o), ref, "e4m3 1024 last step, all (b, h), all rows", _np(lse), ref_lse, _lse_bar(qd, kd, off[s + 1]))
    # the quantisation itself, against the exact attention of the bf16 inputs (a coarse check:
    # e4m3 keeps 3 mantissa bits, so logits move by a few hundredths)
    exact = attention_all_heads(_np(qs), _np(k), _np(v), wl.h, wl.w, s, s + 1)
    qerr = np.abs(_np(o) - exact)
    print(f"[e4m3 vs bf16 inputs] max-abs {qerr.max():.3e} mean-abs {qerr.mean():.3e}", flush=True)
    assert qerr.mean() <= 1e-2


def test_dense_e4m3_whole_and_split_items(api):
    """The 1024px 48x48 step (288 work items) with 6 key splits: on a 256-CU
    device the items of the first round run whole and the rest split.  Every
    row is compared with the unsplit launch (the workspace starts as NaN),
    and rows of heads on both sides of the boundary with the oracle."""
    wl = WORKLOADS["var1024"]
    q, k, v = make_qkv(wl, 74, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    s = 11
    n = off[s + 1] - off[s]
    qs = q[:, :, off[s]:off[s + 1]]
    kc = k[:, :, :off[s + 1]]
    k8, sk = api.var_quantize_e4m3(kc)
    base, base_lse = api.var_attn_dense_e4m3((wl.h, wl.w), qs, k8, sk, v, s, s + 1, return_lse=True)
    ws = api.split_workspace(6, 2, 16, n, 128).fill_(float("nan"))
    o, lse = api.var_attn_dense_e4m3((wl.h, wl.w), qs, k8, sk, v, s, s + 1, return_lse=True, n_splits=6,
                                     workspace=ws)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    d = (o.float() - base.float()).abs()
    print(f"[e4m3 whole+split vs unsplit] max {float(d.max()):.3e} mean {float(d.mean()):.3e}", flush=True)
    assert float(d.max()) <= 1e-2 and float(d.mean()) <= 1e-3
    rows = np.unique(np.concatenate([np.arange(5, n, 71), [n - 1]]))
    for b, h in [(0, 1), (1, 12), (1, 15)]:
        rq, rsq = quantize_tiles(_np(qs[b:b + 1, h:h + 1]))
        rk, rsk = quantize_tiles(_np(kc[b:b + 1, h:h + 1]))
        qd, kd = dequantize_tiles(rq, rsq), dequantize_tiles(rk, rsk)
        ref, ref_lse = oracle.attention(qd, kd, _np(v[b:b + 1, h:h + 1]), wl.h, wl.w, s, s + 1, rows=rows,
                                        return_lse=True)
        _bars(_np(o[b:b + 1, h:h + 1])[:, :, rows], ref, f"e4m3 48x48 x6 b{b} h{h}",
              _np(lse[b:b + 1, h:h + 1])[:, :, rows], ref_lse, _lse_bar(qd, kd, off[s + 1]))
    # two kernel results, each within the bar of the exact LSE: the bar over every (batch, head)
    qd_all = dequantize_tiles(*quantize_tiles(_np(qs)))
    kd_all = dequantize_tiles(*quantize_tiles(_np(kc)))
    assert float((lse - base_lse).abs().max()) <= 2 * _lse_bar(qd_all, kd_all, off[s + 1])


def test_block_sparse_e4m3_shared_and_per_head(api):
    wl = custom_workload(SMALL, 2, 2, 128)
    q, k, v = make_qkv(wl, 74, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    s = 7
    qs = q[:, :, off[s]:off[s + 1]]
    k8, sk, qd, kd = _quantised(api, qs, k)
    mp = api.mask_params(64, 64, 2, 3, 1, 1)
    rp, ci = api.var_build_tile_mask((wl.h, wl.w), s, s + 1, mp)
    kept = oracle.tile_mask(wl.h, wl.w, s, s + 1, 64, 64, 2, 3, 1, 1)
    o, lse = api.var_attn_block_sparse_e4m3((wl.h, wl.w), qs, k8, sk, v, s, s + 1, rp, ci, return_lse=True)
    ref, ref_lse = oracle.attention(qd, kd, _np(v), wl.h, wl.w, s, s + 1, kept=kept, return_lse=True)
    _bars(_np(o), ref, "e4m3 sparse shared", _np(lse), ref_lse, _lse_bar(qd, kd, off[s + 1]))
    # one CSR per (batch, head): random kept tiles per map
    n_qt, n_kt = -(-(off[s + 1] - off[s]) // 64), -(-off[s + 1] // 64)
    rng = np.random.default_rng(75)
    masks = rng.random((4, n_qt, n_kt)) < 0.5
    rps = np.zeros((4, n_qt + 1), np.int32)
    cis = np.zeros((4, n_qt * n_kt), np.int32)
    for m in range(4):
        cols = [np.nonzero(masks[m, r])[0] for r in range(n_qt)]
        rps[m, 1:] = np.cumsum([c.size for c in cols])
        flat = np.concatenate(cols) if rps[m, -1] else np.zeros(0, np.int32)
        cis[m, : flat.size] = flat
    o2, lse2 = api.var_attn_block_sparse_e4m3((wl.h, wl.w), qs, k8, sk, v, s, s + 1,
                                              torch.from_numpy(rps).cuda(), torch.from_numpy(cis).cuda(),
                                              return_lse=True)
    vn = _np(v)
    for m in range(4):
        b, h = divmod(m, 2)
        ref, ref_lse = oracle.attention(qd[b:b + 1, h:h + 1], kd[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1], wl.h, wl.w,
                                        s, s + 1, kept=masks[m], return_lse=True)
        got_lse = _np(lse2[b:b + 1, h:h + 1])
        finite = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(got_lse), finite)
        _bars(_np(o2[b:b + 1, h:h + 1]), ref, f"e4m3 sparse per-head map {m}", got_lse[finite], ref_lse[finite],
              _lse_bar(qd, kd, off[s + 1]))


def test_e4m3_rejects_wrong_dtypes(api):
    wl = custom_workload(SMALL, 1, 1, 128)
    q, k, v = make_qkv(wl, 76, device="cuda")
    k8, sk = api.var_quantize_e4m3(k)
    with pytest.raises(ValueError):
        api.var_attn_dense_e4m3((wl.h, wl.w), q, k, sk, v, 7, 8)          # bf16 keys
    k64 = torch.zeros((1, 1, q.shape[2], 64), dtype=torch.uint8, device="cuda")
    v64 = torch.zeros((1, 1, q.shape[2], 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(api.VarAttnError):
        api.var_attn_dense_e4m3((wl.h, wl.w), v64, k64, sk, v64, 7, 8)    # head_dim 64
