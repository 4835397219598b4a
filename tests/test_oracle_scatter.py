"""Pins for the scatter-restore oracle (CPU only).

With no retained index the result must be torch's nearest interpolation
(library routine); with equal grids and no index it is the identity; with
every index retained it is the update rows placed at their indices; retained
positions are overwritten, never added to ("ARVAR ...", Key Design 3,
Equations (8)-(9)).
"""

import numpy as np
import pytest
import torch

import oracle


@pytest.mark.parametrize("hw_in,hw_out", [((48, 48), (64, 64)), ((3, 5), (7, 9)), ((4, 4), (4, 4)),
                                          ((32, 32), (40, 40)), ((7, 3), (5, 2))])
def test_no_index_is_torch_nearest(hw_in, hw_out):
    (hi, wi), (ho, wo) = hw_in, hw_out
    rng = np.random.default_rng(0)
    base = rng.standard_normal((3, hi * wi, 5)).astype(np.float32)
    out = oracle.scatter_restore(base, hi, wi, np.zeros((3, 0, 5), np.float32), np.zeros(0, np.int32), ho, wo)
    img = torch.from_numpy(base).reshape(3, hi, wi, 5).permute(0, 3, 1, 2)
    ref = torch.nn.functional.interpolate(img, size=(ho, wo), mode="nearest")
    ref = ref.permute(0, 2, 3, 1).reshape(3, ho * wo, 5).numpy()
    assert np.array_equal(out, ref)


def test_equal_grids_no_index_is_identity():
    base = np.random.default_rng(1).standard_normal((2, 30, 4))
    out = oracle.scatter_restore(base, 5, 6, np.zeros((2, 0, 4)), [], 5, 6)
    assert np.array_equal(out, base)


def test_all_indices_place_updates():
    rng = np.random.default_rng(2)
    base = rng.standard_normal((2, 4, 3))
    perm = rng.permutation(16)
    upd = rng.standard_normal((2, 16, 3))
    out = oracle.scatter_restore(base, 2, 2, upd, perm, 4, 4)
    expect = np.empty_like(upd)
    expect[:, perm] = upd
    assert np.array_equal(out, expect)


def test_overwrite_not_add_and_rest_is_base():
    rng = np.random.default_rng(3)
    base = rng.standard_normal((2, 48 * 48, 8)).astype(np.float32) + 10.0
    sel = np.sort(rng.choice(4096, 1638, replace=False)).astype(np.int32)
    upd = rng.standard_normal((2, 1638, 8)).astype(np.float32)
    out = oracle.scatter_restore(base, 48, 48, upd, sel, 64, 64)
    assert np.array_equal(out[:, sel], upd)
    rest = np.setdiff1d(np.arange(4096), sel)
    src = oracle.nearest_source_index(48, 48, 64, 64)
    assert np.array_equal(out[:, rest], base[:, src[rest]])
    # the 48 -> 64 nearest map: destination 4 -> source 3 (floor(4*48/64) = 3)
    assert src[4] == 3 and src[64 * 4] == 48 * 3


def test_bad_indices_raise():
    base = np.zeros((1, 4, 2))
    with pytest.raises(ValueError):
        oracle.scatter_restore(base, 2, 2, np.zeros((1, 2, 2)), [1, 1], 2, 2)
    with pytest.raises(ValueError):
        oracle.scatter_restore(base, 2, 2, np.zeros((1, 1, 2)), [4], 2, 2)
