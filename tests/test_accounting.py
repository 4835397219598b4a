"""Pins for the benchmark's work accounting (CPU only).

The dense counts are checked against closed forms of the schedule: the
visible pairs of a generation are sum_k n_k * L_k (every query of scale k
sees the L_k keys of scales <= k), and a step's traffic is its Q rows, the
K and V prefix once and its O rows.  The sparse count is checked against a
pair-by-pair brute force over the oracle's tile mask, and against the
figures of the 1024px last step (1932 kept tiles, 7,905,984 pairs per
(batch, head)).
"""

import numpy as np

import oracle
from scale_wise_attention_amd import accounting as acc
from scale_wise_attention_amd.inputs import WORKLOADS, custom_workload


def test_dense_generation_pairs_and_flops():
    wl = WORKLOADS["var1024"]
    n = [g * g for g in wl.grids]
    L = np.cumsum(n)
    pairs = int(sum(a * b for a, b in zip(n, L)))
    assert pairs == 68_484_681
    flops = sum(acc.dense_step_flops(wl, s) for s in range(len(n)))
    assert flops == 4.0 * 128 * 2 * 16 * pairs
    # the last step: 4096 queries x 10521 keys
    assert acc.dense_step_flops(wl, 12) == 4.0 * 128 * 32 * 4096 * 10521 == 706_052_358_144
    assert acc.step_sizes(wl.h, wl.w, 12) == (4096, 10521)
    # other schedules of the pages' workloads
    for name, expect in (("var256", 286_434), ("var512", 3_269_850), ("tiny_fp32", 627)):
        w = WORKLOADS[name]
        n = [g * g for g in w.grids]
        assert int(sum(a * b for a, b in zip(n, np.cumsum(n)))) == expect


def test_dense_step_bytes():
    wl = WORKLOADS["var1024"]
    # Q 4096 rows + K and V 10521 rows + O 4096 rows, bf16, 32 (b, h)
    assert acc.dense_step_bytes(wl, 12) == 32 * 128 * 2 * (4096 + 2 * 10521 + 4096) == 239_484_928
    assert acc.dense_step_bytes(wl, 12, out_bytes=4) == 32 * 128 * (4096 * 2 + 2 * 10521 * 2 + 4096 * 4)
    assert acc.dense_step_bytes(wl, 12, rows=1638) == 32 * 128 * 2 * (1638 + 2 * 10521 + 1638)


def _brute_pairs(kept, n_rows, kv_len, t=64):
    pairs = 0
    for i in range(n_rows):
        for u in range(kv_len):
            pairs += bool(kept[i // t, u // t])
    return pairs


def test_sparse_pairs_brute_force():
    rng = np.random.default_rng(3)
    for n_rows, kv_len in ((70, 300), (64, 64), (1, 129), (200, 77)):
        n_qt, n_kt = -(-n_rows // 64), -(-kv_len // 64)
        kept = rng.random((n_qt, n_kt)) < 0.5
        rp, ci = oracle.mask_to_csr(kept)
        assert acc.sparse_pairs(rp, ci, n_rows, kv_len) == _brute_pairs(kept, n_rows, kv_len)


def test_sparse_last_step_1024():
    wl = WORKLOADS["var1024_sparse"]
    kept = oracle.tile_mask(wl.h, wl.w, 12, 13, 64, 64, 7, 7, 2, 2)
    assert int(kept.sum()) == 1932
    rp, ci = oracle.mask_to_csr(kept)
    assert acc.sparse_pairs(rp, ci, 4096, 10521) == 7_905_984
    assert round(acc.sparse_step_flops(wl, rp, ci, 4096, 10521) / 1e9, 2) == 129.53
    # all tiles kept = dense
    full = np.ones_like(kept)
    rp, ci = oracle.mask_to_csr(full)
    assert acc.sparse_step_flops(wl, rp, ci, 4096, 10521) == acc.dense_step_flops(wl, 12)


def test_scatter_bytes():
    assert acc.scatter_bytes(32, 256, 1638, 4096) == 32 * 4096 * 256 * 2
    w = custom_workload([2, 4], 1, 1, 64)
    assert acc.step_sizes(w.h, w.w, 1) == (16, 20)
