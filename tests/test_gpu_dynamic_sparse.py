"""GPU parity of the decision-scale sparse pattern and the per-head sparse attention.

The block mass (a sum of positive attention weights) is compared with the
float64 oracle: given the oracle's LSE, fp32 arithmetic alone (relative
1e-4); given the bf16 attention kernel's LSE (within lse_bound(L) of the
exact one, tests/_bounds.py), relative exp(lse_bound(L)) - 1 + 1e-4.  The
decision tiles and the mapped masks are
integer results: the oracle, applied to the kernel's own float32 masses, must
give them bit for bit.  Attention over per-head masks meets the bf16 bars
(max-abs 1e-2, mean-abs 1e-3).
"""

import numpy as np
import pytest
import torch

import oracle
from _bounds import lse_bound
from oracle.dynamic_sparse import block_mass, decision_tiles, mapped_tile_mask
from scale_wise_attention_amd.inputs import WORKLOADS, make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from scale_wise_attention_amd import api as _api
    return _api


def _np(t):
    return t.detach().float().cpu().numpy()


def _decision_inputs(api, wl, d, seed):
    q, k, v = make_qkv(wl, seed, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    qd = q[:, :, off[d]:off[d + 1]]
    _, lse = api.var_attn_dense((wl.h, wl.w), qd, k, v, d, d + 1, return_lse=True)
    return q, k, v, qd, lse


@pytest.mark.parametrize("wl_name,d", [("var1024", 9), ("var1024", 7), ("var256", 8), ("var512", 6)])
def test_block_mass_matches_oracle(api, wl_name, d):
    wl = WORKLOADS[wl_name]
    q, k, v, qd, lse = _decision_inputs(api, wl, d, 0)
    qn, kn, vn = _np(qd), _np(k), _np(v)
    ref = block_mass(qn, kn, wl.h, wl.w, d)
    _, ref_lse = oracle.attention(qn, kn, vn, wl.h, wl.w, d, d + 1, return_lse=True)
    exact = api.var_attn_block_mass((wl.h, wl.w), qd, k, torch.from_numpy(ref_lse.astype(np.float32)).cuda(), d)
    got = api.var_attn_block_mass((wl.h, wl.w), qd, k, lse, d)
    L = oracle.offsets(wl.h, wl.w)[d + 1]
    for t, bound, what in ((exact, 1e-4, "oracle lse"), (got, np.expm1(lse_bound(L)) + 1e-4, "kernel lse")):
        rel = np.abs(_np(t).astype(np.float64) - ref) / np.maximum(ref, 1e-30)
        print(f"[mass {wl_name} d={d} {what}] max rel {rel.max():.3e}", flush=True)
        assert rel.max() <= bound


@pytest.mark.parametrize("tau", [0.5, 0.9, 0.99, 1.0, 0.0])
def test_decision_tiles_match_oracle_on_kernel_masses(api, tau):
    wl = WORKLOADS["var1024"]
    _, k, _, qd, lse = _decision_inputs(api, wl, 9, 1)
    mass = api.var_attn_block_mass((wl.h, wl.w), qd, k, lse, 9)
    kept = api.var_decision_tiles(mass, tau).cpu().numpy().astype(bool)
    ref = decision_tiles(mass.cpu().numpy(), tau)
    print(f"[decision tau={tau}] kept {kept.mean():.3f}", flush=True)
    assert np.array_equal(kept, ref)


def test_decision_tiles_ties_and_float32_order(api):
    m = np.array([[[0.25, 0.25, 0.25, 0.25], [2.0 ** 24, 1.0, 1.0, 0.0]]], np.float32)
    got = api.var_decision_tiles(torch.from_numpy(m).cuda(), 1.0).cpu().numpy().astype(bool)
    assert np.array_equal(got, decision_tiles(m, 1.0))
    got = api.var_decision_tiles(torch.from_numpy(m).cuda(), 0.5).cpu().numpy().astype(bool)
    assert np.array_equal(got, decision_tiles(m, 0.5))


def _csr_masks(rp, ci, n_kt):
    rp, ci = rp.cpu().numpy(), ci.cpu().numpy()
    return np.stack([oracle.csr_to_mask(rp[m], ci[m, : rp[m, -1]], n_kt) for m in range(rp.shape[0])])


@pytest.mark.parametrize("seed", range(6))
def test_mapped_mask_random_schedules(api, seed):
    rng = np.random.default_rng(1300 + seed)
    K = int(rng.integers(2, 7))
    grids = sorted(int(a) for a in rng.integers(1, 40, K))
    h = grids
    w = sorted(int(a) for a in rng.integers(1, 40, K))
    off = oracle.offsets(h, w)
    d = int(rng.integers(0, K))
    T = int(rng.integers(d, K))
    n_qt_d, n_kt_d = -(-(off[d + 1] - off[d]) // 64), -(-off[d + 1] // 64)
    kept_d = (rng.random((3, n_qt_d, n_kt_d)) < rng.random()).astype(np.uint8)
    rp, ci = api.var_mapped_tile_mask((h, w), d, T, torch.from_numpy(kept_d).cuda())
    ref = mapped_tile_mask(h, w, d, T, kept_d.astype(bool))
    got = _csr_masks(rp, ci, ref.shape[2])
    print(f"[mapped seed {seed}] grids {h}x{w} d={d} T={T} kept {ref.mean():.3f}", flush=True)
    assert np.array_equal(got, ref)


def test_mapped_mask_1024_last_step_from_32x32(api):
    wl = WORKLOADS["var1024"]
    _, k, _, qd, lse = _decision_inputs(api, wl, 9, 2)
    mass = api.var_attn_block_mass((wl.h, wl.w), qd, k, lse, 9)
    kept_d = api.var_decision_tiles(mass, 0.9)
    rp, ci = api.var_mapped_tile_mask((wl.h, wl.w), 9, 12, kept_d)
    kd = kept_d.cpu().numpy().astype(bool).reshape(32, 16, -1)
    sub = [0, 7, 18, 31]
    ref = mapped_tile_mask(wl.h, wl.w, 9, 12, kd[sub])
    got = _csr_masks(rp[sub], ci[sub], ref.shape[2])
    print(f"[mapped 1024] kept {ref.mean():.3f}", flush=True)
    assert np.array_equal(got, ref)
    assert np.array_equal(_csr_masks(rp, ci, ref.shape[2])[sub], ref)


def test_per_head_sparse_attention_matches_oracle(api):
    wl = WORKLOADS["var1024"]
    q, k, v, qd, lse = _decision_inputs(api, wl, 9, 3)
    off = oracle.offsets(wl.h, wl.w)
    mass = api.var_attn_block_mass((wl.h, wl.w), qd, k, lse, 9)
    kept_d = api.var_decision_tiles(mass, 0.9)
    for T in (10, 12):
        rp, ci = api.var_mapped_tile_mask((wl.h, wl.w), 9, T, kept_d)
        qs = q[:, :, off[T]:off[T + 1]]
        o, o_lse = api.var_attn_block_sparse_heads((wl.h, wl.w), qs, k, v, T, T + 1, rp, ci, return_lse=True)
        n = off[T + 1] - off[T]
        rows = np.unique(np.concatenate([np.arange(0, n, 53), [n - 1]]))
        masks = _csr_masks(rp, ci, -(-off[T + 1] // 64))
        qn, kn, vn = _np(qs), _np(k), _np(v)
        for (b, h) in [(0, 4), (1, 11)]:
            m = b * wl.heads + h
            ref, ref_lse = oracle.attention(qn[b:b + 1, h:h + 1], kn[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1],
                                            wl.h, wl.w, T, T + 1, kept=masks[m], rows=rows, return_lse=True)
            err = np.abs(_np(o[b:b + 1, h:h + 1])[:, :, rows] - ref)
            print(f"[per-head T={T} b{b} h{h}] max-abs {err.max():.3e} mean-abs {err.mean():.3e}", flush=True)
            assert err.max() <= 1e-2 and err.mean() <= 1e-3
            assert np.max(np.abs(_np(o_lse[b:b + 1, h:h + 1])[:, :, rows] - ref_lse)) <= lse_bound(off[T + 1])


def test_per_head_csr_equal_maps_match_shared_csr(api):
    """The same CSR for every (batch, head) gives the shared-CSR result bit for bit."""
    wl = WORKLOADS["var1024_sparse"]
    q, k, v = make_qkv(wl, 4, device="cuda")
    off = oracle.offsets(wl.h, wl.w)
    s = 11
    mp = api.mask_params()
    rp, ci = api.var_build_tile_mask((wl.h, wl.w), s, s + 1, mp)
    qs = q[:, :, off[s]:off[s + 1]]
    shared = api.var_attn_block_sparse((wl.h, wl.w), qs, k, v, s, s + 1, rp, ci)
    rps = rp.unsqueeze(0).expand(32, -1).contiguous()
    cis = ci.unsqueeze(0).expand(32, -1).contiguous()
    heads = api.var_attn_block_sparse_heads((wl.h, wl.w), qs, k, v, s, s + 1, rps, cis)
    assert torch.equal(shared, heads)
