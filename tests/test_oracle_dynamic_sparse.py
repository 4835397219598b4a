"""Pins for the decision-scale sparse-pattern oracle (CPU only; readings in
oracle/dynamic_sparse.py).

block_mass: a pure-Python brute force, torch's softmax summed over tiles, row
tiles summing to their row count, and uniform weights.  decision_tiles:
hand-worked cases (order, ties, tau = 0 and 1) and one that only float32 sums
decide.  mapped_tile_mask: a pure-Python pair enumeration, the identity when
the decision scale is the step itself, and an all-kept decision.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.dynamic_sparse import block_mass, decision_tiles, mapped_tile_mask


def _py_mass(q, k, h, w, d, tile):
    off = oracle.offsets(h, w)
    L, n = off[d + 1], off[d + 1] - off[d]
    B, H, _, D = q.shape
    scale = 1.0 / math.sqrt(D)
    n_qt, n_kt = -(-n // tile), -(-L // tile)
    out = np.zeros((B, H, n_qt, n_kt))
    for b in range(B):
        for hh in range(H):
            acc = [[[] for _ in range(n_kt)] for _ in range(n_qt)]
            for i in range(n):
                lg = [scale * math.fsum(float(q[b, hh, i, e]) * float(k[b, hh, u, e]) for e in range(D)) for u in range(L)]
                m = max(lg)
                ex = [math.exp(a - m) for a in lg]
                tot = math.fsum(ex)
                for u in range(L):
                    acc[i // tile][u // tile].append(ex[u] / tot)
            for r in range(n_qt):
                for c in range(n_kt):
                    out[b, hh, r, c] = math.fsum(acc[r][c])
    return out


@pytest.mark.parametrize("seed", range(4))
def test_block_mass_matches_python_brute_force(seed):
    rng = np.random.default_rng(900 + seed)
    K = int(rng.integers(2, 5))
    h = [int(a) for a in rng.integers(1, 5, K)]
    w = [int(a) for a in rng.integers(1, 5, K)]
    off = oracle.offsets(h, w)
    d = int(rng.integers(0, K))
    tile = int(rng.integers(1, 6))
    q = rng.standard_normal((1, 2, off[d + 1] - off[d], 4))
    k = rng.standard_normal((1, 2, off[K], 4))
    got = block_mass(q, k, h, w, d, tile=tile)
    assert np.max(np.abs(got - _py_mass(q, k, h, w, d, tile))) <= 1e-12


def test_block_mass_is_torch_softmax_summed_over_tiles_and_rows_sum_to_counts():
    h = w = [1, 2, 4, 6, 8]
    off = oracle.offsets(h, w)
    rng = np.random.default_rng(11)
    d = 4
    q = rng.standard_normal((2, 2, 64, 16))
    k = rng.standard_normal((2, 2, off[5], 16))
    got = block_mass(q, k, h, w, d, tile=16)
    p = torch.softmax(torch.from_numpy(q) @ torch.from_numpy(k[:, :, :off[5]]).transpose(-1, -2) / 4.0, dim=-1)
    L = off[5]
    pad = torch.nn.functional.pad(p, (0, 16 * (-(-L // 16)) - L))
    ref = pad.reshape(2, 2, 4, 16, -1, 16).sum(dim=(3, 5)).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-12
    assert np.max(np.abs(got.sum(axis=-1) - 16.0)) <= 1e-12


def test_block_mass_uniform_weights():
    h = w = [1, 2, 3, 4]
    off = oracle.offsets(h, w)
    L = off[4]
    k = np.broadcast_to(np.random.default_rng(3).standard_normal(8), (1, 1, L, 8)).copy()
    q = np.random.default_rng(4).standard_normal((1, 1, 16, 8))
    got = block_mass(q, k, h, w, 3, tile=4)
    sizes = np.array([min(4, L - 4 * c) for c in range(-(-L // 4))])
    assert np.max(np.abs(got[0, 0] - 4 * sizes[None, :] / L)) <= 1e-14


def test_decision_tiles_hand_cases():
    m = np.array([[0.5, 0.3, 0.2]], np.float32)
    assert decision_tiles(m, 0.6).tolist() == [[True, True, False]]
    assert decision_tiles(m, 0.5).tolist() == [[True, False, False]]
    assert decision_tiles(m, 0.0).tolist() == [[False, False, False]]
    assert decision_tiles(np.array([[0.2, 0.3, 0.5]], np.float32), 0.6).tolist() == [[False, True, True]]
    ties = np.array([[0.25, 0.25, 0.25, 0.25]], np.float32)
    assert decision_tiles(ties, 0.5).tolist() == [[True, True, False, False]]      # equal masses: lower c first
    exact = np.array([[0.5, 0.25, 0.25, 0.0]], np.float32)
    assert decision_tiles(exact, 1.0).tolist() == [[True, True, True, False]]
    # float32: 2^24 + 1 rounds to 2^24, so the total is 2^24 and one tile already reaches it
    big = np.array([[2.0 ** 24, 1.0, 1.0]], np.float32)
    assert decision_tiles(big, 1.0).tolist() == [[True, False, False]]
    assert decision_tiles(np.zeros((2, 3, 5), np.float32), 0.9).shape == (2, 3, 5)


def _py_mapped(h, w, d, T, kept_d, tile):
    off = oracle.offsets(h, w)

    def coords(t):
        s = max(j for j in range(len(h)) if off[j] <= t)
        return s, (t - off[s]) // w[s], (t - off[s]) % w[s]

    L, n = off[T + 1], off[T + 1] - off[T]
    out = np.zeros((kept_d.shape[0], -(-n // tile), -(-L // tile)), dtype=bool)
    for m in range(kept_d.shape[0]):
        for i in range(n):
            _, yq, xq = coords(off[T] + i)
            r = ((yq * h[d]) // h[T] * w[d] + (xq * w[d]) // w[T]) // tile
            for u in range(L):
                j, yu, xu = coords(u)
                ud = u if j <= d else off[d] + (yu * h[d]) // h[j] * w[d] + (xu * w[d]) // w[j]
                if kept_d[m, r, ud // tile]:
                    out[m, i // tile, u // tile] = True
    return out


@pytest.mark.parametrize("seed", range(6))
def test_mapped_mask_matches_python_pair_enumeration(seed):
    rng = np.random.default_rng(950 + seed)
    K = int(rng.integers(2, 5))
    h = sorted(int(a) for a in rng.integers(1, 7, K))
    w = sorted(int(a) for a in rng.integers(1, 7, K))
    off = oracle.offsets(h, w)
    d = int(rng.integers(0, K))
    T = int(rng.integers(d, K))
    tile = int(rng.integers(1, 6))
    n_d = off[d + 1] - off[d]
    kept_d = rng.random((2, -(-n_d // tile), -(-off[d + 1] // tile))) < 0.4
    assert np.array_equal(mapped_tile_mask(h, w, d, T, kept_d, tile), _py_mapped(h, w, d, T, kept_d, tile))


def test_mapped_mask_identity_at_the_decision_scale_and_all_kept():
    h = w = [1, 2, 4, 6, 8]
    off = oracle.offsets(h, w)
    rng = np.random.default_rng(12)
    kept_d = rng.random((3, 4, -(-off[5] // 16))) < 0.3
    assert np.array_equal(mapped_tile_mask(h, w, 4, 4, kept_d, 16), kept_d)
    h2 = w2 = [1, 2, 4, 6, 8, 12]
    full = np.ones((1, 4, -(-off[5] // 16)), dtype=bool)
    got = mapped_tile_mask(h2, w2, 4, 5, full, 16)
    assert got.all() and got.shape == (1, 9, -(-oracle.offsets(h2, w2)[6] // 16))
