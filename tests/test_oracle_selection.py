"""Pins for the attention-guided selection oracle (CPU only).

Saliency ("ARVAR ...", Key Design 2; readings in oracle/selection.py) is
checked against a pure-Python brute force on tiny schedules, torch's softmax
on a one-scale schedule, and closed forms (uniform weights give 1/L, a single
token gives 1, the total equals the mean own-scale mass of the attention
weights).  The Top-K choice is checked against a brute-force sort, ties
(lowest position first), the n_keep edge cases, numpy's argsort on distinct
scores, and a case where only float32 in-order summation of the maps gives
the documented answer.
"""

import math

import numpy as np
import pytest
import torch

import oracle


def _py_saliency(q, k, h, w, step, scale):
    off = oracle.offsets(h, w)
    L, n_s = off[step + 1], off[step + 1] - off[step]
    B, H = q.shape[:2]
    out = np.zeros((B, H, n_s))
    for b in range(B):
        for hh in range(H):
            cols = [[] for _ in range(n_s)]
            for i in range(n_s):
                lg = [scale * math.fsum(float(q[b, hh, i, d]) * float(k[b, hh, u, d]) for d in range(q.shape[3]))
                      for u in range(L)]
                m = max(lg)
                ex = [math.exp(x - m) for x in lg]
                tot = math.fsum(ex)
                for u in range(n_s):
                    cols[u].append(ex[off[step] + u] / tot)
            for u in range(n_s):
                out[b, hh, u] = math.fsum(cols[u]) / n_s
    return out


@pytest.mark.parametrize("seed", range(6))
def test_saliency_matches_python_brute_force(seed):
    rng = np.random.default_rng(300 + seed)
    K = int(rng.integers(1, 5))
    h = [int(a) for a in rng.integers(1, 5, K)]
    w = [int(a) for a in rng.integers(1, 5, K)]
    off = oracle.offsets(h, w)
    step = int(rng.integers(0, K))
    D = int(rng.integers(1, 9))
    q = rng.standard_normal((1, 2, off[step + 1] - off[step], D))
    k = rng.standard_normal((1, 2, off[K], D))
    got = oracle.saliency(q, k, h, w, step)
    ref = _py_saliency(q, k, h, w, step, 1.0 / math.sqrt(D))
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_saliency_one_scale_is_torch_softmax_column_mean():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((2, 3, 35, 16))
    k = rng.standard_normal((2, 3, 35, 16))
    got = oracle.saliency(q, k, [5], [7], 0, softmax_scale=0.3)
    p = torch.softmax(0.3 * torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2), dim=-1)
    ref = p.mean(dim=-2).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-14
    assert np.max(np.abs(got.sum(axis=-1) - 1.0)) <= 1e-12     # every row's mass is on its own scale


def test_saliency_uniform_weights_give_one_over_L():
    h = w = [1, 2, 3, 4]
    off = oracle.offsets(h, w)
    rng = np.random.default_rng(8)
    k_same = np.broadcast_to(rng.standard_normal(8), (1, 2, off[4], 8)).copy()      # identical keys
    q = rng.standard_normal((1, 2, 16, 8))
    got = oracle.saliency(q, k_same, h, w, 3)
    assert np.max(np.abs(got - 1.0 / off[4])) <= 1e-15
    got0 = oracle.saliency(np.zeros((1, 2, 9, 8)), rng.standard_normal((1, 2, off[4], 8)), h, w, 2)  # zero queries
    assert np.max(np.abs(got0 - 1.0 / off[3])) <= 1e-15


def test_saliency_single_token_scale_is_one():
    rng = np.random.default_rng(9)
    got = oracle.saliency(rng.standard_normal((2, 2, 1, 4)), rng.standard_normal((2, 2, 30, 4)), [1, 2, 5], [1, 2, 5], 0)
    assert np.array_equal(got, np.ones((2, 2, 1)))


def test_saliency_total_is_mean_own_scale_mass_of_attention_weights():
    h = w = [1, 2, 3, 5]
    off = oracle.offsets(h, w)
    rng = np.random.default_rng(10)
    q = rng.standard_normal((1, 2, off[4] - off[3], 12))
    k = rng.standard_normal((1, 2, off[4], 12))
    v = rng.standard_normal((1, 2, off[4], 12))
    _, p = oracle.attention(q, k, v, h, w, 3, 4, return_probs=True)
    got = oracle.saliency(q, k, h, w, 3)
    assert np.max(np.abs(got.sum(axis=-1) - p[..., off[3]:].sum(axis=-1).mean(axis=-1))) <= 1e-13
    assert np.max(np.abs(got - p[..., off[3]:].mean(axis=-2))) <= 1e-15


def _brute_select(maps, hs, ws, hd, wd, n_keep):
    maps = np.asarray(maps, dtype=np.float32)
    score = []
    for t in range(hd * wd):
        y, x = divmod(t, wd)
        src = (y * hs // hd) * ws + (x * ws // wd)
        acc = np.float32(0.0)
        for m in range(maps.shape[0]):
            acc = np.float32(acc + maps[m, src])
        score.append(float(acc))
    best = sorted(range(hd * wd), key=lambda t: (-score[t], t))[:n_keep]
    return sorted(best)


@pytest.mark.parametrize("seed", range(10))
def test_select_matches_brute_force_sort(seed):
    rng = np.random.default_rng(400 + seed)
    hs, ws = int(rng.integers(1, 9)), int(rng.integers(1, 9))
    hd, wd = hs + int(rng.integers(0, 9)), ws + int(rng.integers(0, 9))
    maps = np.round(rng.random((int(rng.integers(1, 5)), hs * ws)) * 4) / 4          # many ties
    n_keep = int(rng.integers(0, hd * wd + 1))
    got = oracle.select_positions(maps.astype(np.float32), hs, ws, hd, wd, n_keep)
    assert got.dtype == np.int32
    assert got.tolist() == _brute_select(maps, hs, ws, hd, wd, n_keep)


def test_select_ties_keep_lowest_positions_and_edges():
    maps = np.full((3, 12), 0.25, np.float32)
    assert oracle.select_positions(maps, 3, 4, 6, 8, 10).tolist() == list(range(10))
    assert oracle.select_positions(maps, 3, 4, 6, 8, 0).size == 0
    assert oracle.select_positions(maps, 3, 4, 6, 8, 48).tolist() == list(range(48))
    with pytest.raises(ValueError):
        oracle.select_positions(maps, 3, 4, 6, 8, 49)


def test_select_distinct_scores_same_grid_is_argsort():
    rng = np.random.default_rng(11)
    maps = rng.random((1, 64)).astype(np.float32)
    got = oracle.select_positions(maps, 8, 8, 8, 8, 20)
    assert got.tolist() == sorted(np.argsort(-maps[0], kind="stable")[:20].tolist())


def test_select_sums_maps_in_float32_in_order():
    # in float32, 2^24 + 1 rounds back to 2^24: position 0 scores 2^24 and
    # position 1 scores 2^24 + 2; an exact sum would tie them (position 0 first)
    maps = np.array([[2.0 ** 24, 2.0 ** 24], [1.0, 0.0], [1.0, 2.0]], np.float32)
    assert oracle.select_positions(maps, 1, 2, 1, 2, 1).tolist() == [1]
    assert oracle.selection_scores(maps, 1, 2, 1, 2).tolist() == [2.0 ** 24, 2.0 ** 24 + 2]
