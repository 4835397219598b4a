"""Pins for the attention oracle (CPU only).

The pages print no attention inputs or outputs, so the oracle is pinned by
things other than itself:

* a pair-by-pair pure-Python brute force (math.fsum / math.exp) on tiny
  schedules, with the visibility decided by walking the grids token by token;
* invariants that follow from the definition (single-key rows return v
  exactly, identical keys give the mean of V, row weights sum to 1, a sparse
  run with every tile kept is the dense run);
* library routines: torch's scaled_dot_product_attention on the CPU in
  float64 (unmasked for a one-scale schedule, with an explicit boolean mask
  otherwise) and scipy's logsumexp for the LSE;
* the closed form sum_k n_k * L_k for the number of visible pairs.
"""

import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from scale_wise_attention_amd.inputs import WORKLOADS, make_qkv_f32


def _tokens_by_walking(h, w):
    """[(scale, y, x)] for every token, built by visiting the grids in order."""
    toks = []
    for s in range(len(h)):
        for yy in range(h[s]):
            for xx in range(w[s]):
                toks.append((s, yy, xx))
    return toks


def brute_force(q, k, v, h, w, qb, qe, scale, q_index=None, kept=None, tile_q=64, tile_k=64):
    """Pair-by-pair attention with Python floats and math.fsum."""
    toks = _tokens_by_walking(h, w)
    first = sum(h[s] * w[s] for s in range(qb))
    L = sum(h[s] * w[s] for s in range(qe))
    n_q = L - first
    pos = list(range(n_q)) if q_index is None else [int(i) for i in q_index]
    B, H, _, D = q.shape
    out = np.zeros((B, H, len(pos), D))
    for bi in range(B):
        for hi in range(H):
            for row, p in enumerate(pos):
                t = first + p
                keys = []
                for u in range(L):
                    if toks[u][0] > toks[t][0]:
                        continue
                    if kept is not None and not kept[row // tile_q][u // tile_k]:
                        continue
                    keys.append(u)
                if not keys:
                    continue
                logits = [scale * math.fsum(float(q[bi, hi, p, d]) * float(k[bi, hi, u, d]) for d in range(D))
                          for u in keys]
                m = max(logits)
                ps = [math.exp(s - m) for s in logits]
                l = math.fsum(ps)
                for d in range(D):
                    out[bi, hi, row, d] = math.fsum(pp * float(v[bi, hi, u, d]) for pp, u in zip(ps, keys)) / l
    return out


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_brute_force_tiny_workload_full_sequence():
    wl = WORKLOADS["tiny_fp32"]
    q, k, v = make_qkv_f32(wl, seed=0)
    got = oracle.attention(q, k, v, wl.h, wl.w, 0, wl.num_scales)
    ref = brute_force(q, k, v, wl.h, wl.w, 0, wl.num_scales, 1 / math.sqrt(wl.head_dim))
    assert np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_random_schedules(seed):
    rng = np.random.default_rng(100 + seed)
    K = int(rng.integers(1, 5))
    h = [int(a) for a in rng.integers(1, 5, K)]
    w = [int(a) for a in rng.integers(1, 5, K)]
    D = int(rng.integers(1, 9))
    L = sum(a * b for a, b in zip(h, w))
    q = _rand((1, 2, L, D), seed)
    k = _rand((1, 2, L, D), seed + 50)
    v = _rand((1, 2, L, D), seed + 99)
    qb = int(rng.integers(0, K))
    qe = int(rng.integers(qb + 1, K + 1))
    first = sum(a * b for a, b in zip(h[:qb], w[:qb]))
    n_q = sum(a * b for a, b in zip(h[:qe], w[:qe])) - first
    qblock = q[:, :, first:first + n_q]
    scale = 0.37
    # plain
    got = oracle.attention(qblock, k, v, h, w, qb, qe, softmax_scale=scale)
    ref = brute_force(qblock, k, v, h, w, qb, qe, scale)
    assert np.max(np.abs(got - ref)) <= 1e-12
    # gathered rows, in a scrambled order
    sel = rng.permutation(n_q)[: max(1, n_q // 2)]
    got = oracle.attention(qblock, k, v, h, w, qb, qe, softmax_scale=scale, q_index=sel)
    ref = brute_force(qblock, k, v, h, w, qb, qe, scale, q_index=sel)
    assert np.max(np.abs(got - ref)) <= 1e-12
    # a random tile mask with tile size 2 (column 0 always kept so no row is empty)
    tq, tk = 2, 2
    n_qt, n_kt = -(-n_q // tq), -(-sum(a * b for a, b in zip(h[:qe], w[:qe])) // tk)
    kept = rng.random((n_qt, n_kt)) < 0.5
    kept[:, 0] = True
    got = oracle.attention(qblock, k, v, h, w, qb, qe, softmax_scale=scale, kept=kept, tile_q=tq, tile_k=tk)
    ref = brute_force(qblock, k, v, h, w, qb, qe, scale, kept=kept, tile_q=tq, tile_k=tk)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_first_scale_query_returns_v0_exactly():
    wl = WORKLOADS["var256"]
    q, k, v = make_qkv_f32(wl, seed=3)
    q, k, v = q[:, :2], k[:, :2], v[:, :2]
    o_full = oracle.attention(q, k, v, wl.h, wl.w, 0, wl.num_scales, rows=[0, 1, 2])
    assert np.array_equal(o_full[:, :, 0, :], v[:, :, 0, :].astype(np.float64))
    o_step = oracle.attention(q[:, :, :1], k, v, wl.h, wl.w, 0, 1)
    assert np.array_equal(o_step[:, :, 0, :], v[:, :, 0, :].astype(np.float64))


def test_identical_keys_give_mean_of_visible_values():
    h, w = [1, 2, 3], [1, 2, 3]
    L = 14
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 3, L, 8))
    k = np.broadcast_to(rng.standard_normal(8), (2, 3, L, 8)).copy()
    v = rng.standard_normal((2, 3, L, 8))
    o = oracle.attention(q, k, v, h, w, 0, 3)
    ends = [1, 5, 14]
    scale_of = [0] + [1] * 4 + [2] * 9
    for t in range(L):
        mean = v[:, :, : ends[scale_of[t]], :].mean(axis=2)
        assert np.max(np.abs(o[:, :, t] - mean)) <= 1e-12


def test_row_weights_sum_to_one_and_lse_matches_logsumexp():
    wl = WORKLOADS["tiny_fp32"]
    q, k, v = make_qkv_f32(wl, seed=1)
    o, lse, p = oracle.attention(q, k, v, wl.h, wl.w, 0, 4, return_lse=True, return_probs=True)
    assert np.max(np.abs(p.sum(axis=-1) - 1.0)) <= 1e-12
    # lse against scipy on explicitly written masked logits
    scale = 1 / math.sqrt(32)
    ends = [1, 5, 14, 30]
    scale_of = [0] + [1] * 4 + [2] * 9 + [3] * 16
    for bi in range(1):
        for hi in range(2):
            for t in range(30):
                s = scale * (q[bi, hi, t].astype(np.float64) @ k[bi, hi, : ends[scale_of[t]]].astype(np.float64).T)
                assert abs(lse[bi, hi, t] - logsumexp(s)) <= 1e-12


def test_visible_pair_count_closed_form():
    """#visible pairs of a full-sequence run equals sum_k n_k * L_k."""
    for name in ("tiny_fp32", "var256", "var512"):
        wl = WORKLOADS[name]
        sizes = [g * g for g in wl.grids]
        closed = sum(n * sum(sizes[: i + 1]) for i, n in enumerate(sizes))
        L = sum(sizes)
        rng = np.random.default_rng(0)
        # small D and one head keep this fast; the weights are > 0 exactly where visible
        q = rng.standard_normal((1, 1, L, 2)) * 0.1
        k = rng.standard_normal((1, 1, L, 2)) * 0.1
        v = rng.standard_normal((1, 1, L, 2))
        _, p = oracle.attention(q, k, v, wl.h, wl.w, 0, wl.num_scales, return_probs=True)
        assert int((p > 0).sum()) == closed
    assert closed == 3269850  # value for the 512px schedule


def test_one_scale_schedule_is_unmasked_sdpa():
    rng = np.random.default_rng(9)
    h, w = [5], [7]
    q = rng.standard_normal((2, 3, 35, 16))
    k = rng.standard_normal((2, 3, 35, 16))
    v = rng.standard_normal((2, 3, 35, 16))
    got = oracle.attention(q, k, v, h, w, 0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-12


def _block_causal_bool(h, w):
    toks = _tokens_by_walking(h, w)
    L = len(toks)
    m = np.zeros((L, L), dtype=bool)
    for t in range(L):
        for u in range(L):
            m[t, u] = toks[u][0] <= toks[t][0]
    return m


def test_full_sequence_is_sdpa_with_block_causal_mask():
    wl = WORKLOADS["var256"]
    q, k, v = make_qkv_f32(wl, seed=2)
    q, k, v = q[:1, :2], k[:1, :2], v[:1, :2]
    got = oracle.attention(q, k, v, wl.h, wl.w, 0, wl.num_scales)
    mask = torch.from_numpy(_block_causal_bool(wl.h, wl.w))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64)), torch.from_numpy(k.astype(np.float64)),
        torch.from_numpy(v.astype(np.float64)), attn_mask=mask).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_sparse_is_sdpa_with_expanded_tile_mask_and_all_kept_equals_dense():
    wl = WORKLOADS["var256"]
    q, k, v = make_qkv_f32(wl, seed=4)
    q, k, v = q[:1, :2], k[:1, :2], v[:1, :2]
    h, w = wl.h, wl.w
    L = wl.tokens
    tq = tk = 16
    kept = oracle.tile_mask(h, w, 0, wl.num_scales, tq, tk, sink_scales=3, local_from_scale=3,
                            radius_y=1, radius_x=1)
    row_ptr, col_idx = oracle.mask_to_csr(kept)
    # expand the CSR by hand into a token mask
    allowed = np.zeros((L, L), dtype=bool)
    for r in range(len(row_ptr) - 1):
        for c in col_idx[row_ptr[r]:row_ptr[r + 1]]:
            allowed[r * tq:(r + 1) * tq, c * tk:(c + 1) * tk] = True
    mask = torch.from_numpy(_block_causal_bool(h, w) & allowed)
    got = oracle.attention(q, k, v, h, w, 0, wl.num_scales, kept=kept, tile_q=tq, tile_k=tk)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64)), torch.from_numpy(k.astype(np.float64)),
        torch.from_numpy(v.astype(np.float64)), attn_mask=mask).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-12
    # every tile kept: bit-identical to the dense oracle
    all_kept = np.ones_like(kept)
    dense = oracle.attention(q, k, v, h, w, 0, wl.num_scales)
    sparse = oracle.attention(q, k, v, h, w, 0, wl.num_scales, kept=all_kept, tile_q=tq, tile_k=tk)
    assert np.array_equal(dense, sparse)


def test_step_mode_equals_rows_of_full_sequence():
    wl = WORKLOADS["var256"]
    q, k, v = make_qkv_f32(wl, seed=6)
    q, k, v = q[:1, :2], k[:1, :2], v[:1, :2]
    full = oracle.attention(q, k, v, wl.h, wl.w, 0, wl.num_scales)
    off = oracle.offsets(wl.h, wl.w)
    for s in range(wl.num_scales):
        step = oracle.attention(q[:, :, off[s]:off[s + 1]], k, v, wl.h, wl.w, s, s + 1)
        assert np.max(np.abs(step - full[:, :, off[s]:off[s + 1]])) <= 1e-12


def test_rows_subset_and_gather_match_full_rows():
    wl = WORKLOADS["var256"]
    q, k, v = make_qkv_f32(wl, seed=8)
    q, k, v = q[:1, :1], k[:1, :1], v[:1, :1]
    off = oracle.offsets(wl.h, wl.w)
    qb = q[:, :, off[9]:off[10]]
    full = oracle.attention(qb, k, v, wl.h, wl.w, 9, 10)
    sel = np.array([255, 3, 17, 100], dtype=np.int32)
    g = oracle.attention(qb, k, v, wl.h, wl.w, 9, 10, q_index=sel)
    assert np.max(np.abs(g[0, 0] - full[0, 0, sel])) <= 1e-12
    r = oracle.attention(qb, k, v, wl.h, wl.w, 9, 10, rows=[7, 200])
    assert np.max(np.abs(r[0, 0] - full[0, 0, [7, 200]])) <= 1e-12


def test_row_without_visible_key_is_zero_with_neg_inf_lse():
    h, w = [2], [2]
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 1, 4, 4))
    kept = np.array([[False]])
    o, lse = oracle.attention(q, q, q, h, w, 0, 1, kept=kept, tile_q=4, tile_k=4, return_lse=True)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
