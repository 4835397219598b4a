"""Pins for the tile-mask oracle (CPU only).

Pinned by hand derivations (tests/golden), closed forms of special cases
(a single scale reduces to a Chebyshev neighbourhood; an exact 2x grid ratio
reduces to halving coordinates; sinks alone keep exactly the sink columns; a
window wider than every grid keeps every visible tile) and structural
properties (monotone in the radius, gathering all rows in order changes
nothing, CSR round trip).
"""

import os

import numpy as np
import pytest

import oracle
from scale_wise_attention_amd.inputs import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def test_hand_derived_tiny_mask():
    rows = _read_rows("tile_mask_tiny.txt")
    expect = np.array([[c == "1" for c in r] for r in rows])
    got = oracle.tile_mask([1, 2, 3, 4], [1, 2, 3, 4], 0, 4, tile_q=4, tile_k=4,
                           sink_scales=1, local_from_scale=1, radius_y=0, radius_x=0)
    assert got.shape == (8, 8)
    assert np.array_equal(got, expect)


def test_hand_derived_1024_last_step_row0():
    expect = [int(a) for a in _read_rows("tile_mask_1024_row0.txt")[0].split()]
    wl = WORKLOADS["var1024_sparse"]
    K = wl.num_scales
    # only the first query tile is needed: pass its 64 positions as the query set
    got = oracle.tile_mask(wl.h, wl.w, K - 1, K, 64, 64, 7, 7, 2, 2, q_index=np.arange(64))
    assert list(np.nonzero(got[0])[0]) == expect


def test_hand_derived_1024_last_step_row63():
    expect = [int(a) for a in _read_rows("tile_mask_1024_row63.txt")[0].split()]
    wl = WORKLOADS["var1024_sparse"]
    K = wl.num_scales
    # the last query tile: the 64 positions of grid row 63
    got = oracle.tile_mask(wl.h, wl.w, K - 1, K, 64, 64, 7, 7, 2, 2, q_index=np.arange(4032, 4096))
    assert list(np.nonzero(got[0])[0]) == expect


def test_1024_generation_mask_figures():
    """Figures of the 1024px sparse workload's masks from an independent pair-by-pair
    enumeration written for the workload description (not from the pages, which print
    none), under the same readings (literal index map compared by cross-multiplication,
    tiles aligned at the call's first row and at key token 0, real visible pairs only).
    They pin the window rule on far rows and on every step, not only row 0 and the total."""
    from scale_wise_attention_amd import accounting as acc
    wl = WORKLOADS["var1024_sparse"]
    K = wl.num_scales
    off = oracle.offsets(wl.h, wl.w)
    kept_total = {7: (80, 105), 8: (136, 216), 9: (284, 640), 10: (525, 1625), 11: (915, 3636),
                  12: (1932, 10560)}
    pairs = 0
    for s in range(K):
        kept = oracle.tile_mask(wl.h, wl.w, s, s + 1, 64, 64, 7, 7, 2, 2)
        if s < 7:
            assert kept.all(), f"step {s}: steps of sink scales only keep every tile"
        else:
            assert (int(kept.sum()), kept.size) == kept_total[s], f"step {s}"
        rp, ci = oracle.mask_to_csr(kept)
        pairs += acc.sparse_pairs(rp, ci, off[s + 1] - off[s], off[s + 1])
        if s == K - 1:
            nnz = np.diff(rp)
            assert (int(nnz.min()), int(nnz.max())) == (24, 33)
            assert int(ci.sum()) == 95_967
            assert int(sum((r + 1) * int(ci[rp[r]:rp[r + 1]].sum()) for r in range(rp.size - 1))) == 3_349_961
    # computed (visible, kept) pairs of the whole sparse generation: 23.3 % of the dense 68,484,681
    assert pairs == 15_977_033


@pytest.mark.parametrize("R", [0, 1, 2])
def test_single_scale_tile1_is_chebyshev_neighbourhood(R):
    h, w = [5], [6]
    got = oracle.tile_mask(h, w, 0, 1, 1, 1, sink_scales=0, local_from_scale=0, radius_y=R, radius_x=R)
    for i in range(30):
        for u in range(30):
            near = abs(i // 6 - u // 6) <= R and abs(i % 6 - u % 6) <= R
            assert got[i, u] == near


def test_exact_half_resolution_maps_by_halving():
    # grids 2x2 then 4x4; a 4x4 query at (y, x) maps to (y/2, x/2) in the 2x2 grid
    h = w = [2, 4]
    got = oracle.tile_mask(h, w, 1, 2, 1, 1, sink_scales=0, local_from_scale=0, radius_y=0, radius_x=0)
    for i in range(16):
        yq, xq = divmod(i, 4)
        for u in range(4):
            yk, xk = divmod(u, 2)
            expect = (yq == 2 * yk) and (xq == 2 * xk)
            assert got[i, u] == expect
    # radius 1: |y_q/2 - y_k| <= 1
    got = oracle.tile_mask(h, w, 1, 2, 1, 1, sink_scales=0, local_from_scale=0, radius_y=1, radius_x=1)
    for i in range(16):
        yq, xq = divmod(i, 4)
        for u in range(4):
            yk, xk = divmod(u, 2)
            assert got[i, u] == (abs(yq - 2 * yk) <= 2 and abs(xq - 2 * xk) <= 2)


def test_sinks_alone_keep_exactly_the_sink_columns_in_step_mode():
    wl = WORKLOADS["var1024_sparse"]
    K = wl.num_scales
    off = oracle.offsets(wl.h, wl.w)
    got = oracle.tile_mask(wl.h, wl.w, K - 2, K - 1, 64, 64, sink_scales=7, local_from_scale=K,
                           radius_y=2, radius_x=2)
    n_sink_tiles = -(-off[7] // 64)
    expect = np.zeros_like(got)
    expect[:, :n_sink_tiles] = True
    assert np.array_equal(got, expect)


def test_huge_window_keeps_every_visible_tile():
    wl = WORKLOADS["var256"]
    h, w = wl.h, wl.w
    got = oracle.tile_mask(h, w, 0, wl.num_scales, 16, 16, sink_scales=0, local_from_scale=0,
                           radius_y=100, radius_x=100)
    # tile-level block-causal visibility written independently
    scale_of = []
    for s, g in enumerate(wl.grids):
        scale_of += [s] * (g * g)
    L = len(scale_of)
    expect = np.zeros((-(-L // 16), -(-L // 16)), dtype=bool)
    for t in range(L):
        for u in range(L):
            if scale_of[u] <= scale_of[t]:
                expect[t // 16, u // 16] = True
    assert np.array_equal(got, expect)


def test_monotone_in_radius_and_sink_tiles_always_present():
    wl = WORKLOADS["var512"]
    K = wl.num_scales
    off = oracle.offsets(wl.h, wl.w)
    prev = None
    for R in range(4):
        m = oracle.tile_mask(wl.h, wl.w, K - 1, K, 64, 64, sink_scales=3, local_from_scale=3,
                             radius_y=R, radius_x=R)
        assert m[:, : -(-off[3] // 64)].all()
        if prev is not None:
            assert np.all(m | ~prev) and (m.sum() >= prev.sum())
        prev = m


def test_gathering_all_rows_in_order_changes_nothing_and_csr_round_trip():
    wl = WORKLOADS["var512"]
    K = wl.num_scales
    a = oracle.tile_mask(wl.h, wl.w, K - 2, K, 32, 64, 3, 3, 2, 2)
    n_q = oracle.offsets(wl.h, wl.w)[K] - oracle.offsets(wl.h, wl.w)[K - 2]
    b = oracle.tile_mask(wl.h, wl.w, K - 2, K, 32, 64, 3, 3, 2, 2, q_index=np.arange(n_q))
    assert np.array_equal(a, b)
    rp, ci = oracle.mask_to_csr(a)
    assert rp[0] == 0 and rp[-1] == ci.size and rp.dtype == np.int32 and ci.dtype == np.int32
    for r in range(a.shape[0]):
        row = ci[rp[r]:rp[r + 1]]
        assert np.all(np.diff(row) > 0)
    assert np.array_equal(oracle.csr_to_mask(rp, ci, a.shape[1]), a)


def test_pruned_rows_are_subsets_of_their_positions_masks():
    """A query row's own selected key tiles do not depend on which rows share its tile."""
    wl = WORKLOADS["var512"]
    K = wl.num_scales
    sel = np.array([5, 70, 400, 1000], dtype=np.int64)
    per_row = oracle.tile_mask(wl.h, wl.w, K - 1, K, 1, 64, 3, 3, 2, 2, q_index=sel)
    together = oracle.tile_mask(wl.h, wl.w, K - 1, K, 4, 64, 3, 3, 2, 2, q_index=sel)
    assert np.array_equal(together[0], per_row.any(axis=0))
