"""Pins for the e4m3 quantisation oracle (CPU only).

The encoder is checked against torch's float8_e4m3fn cast (a library
routine, round to nearest even) on random values, ties, subnormals and the
largest codes; decoding inverts encoding on every finite code; the map
scales reproduce amax / 448 and every map's largest magnitude quantises to
448; tile groups are independent of each other and a whole-map call on a
tile-sized tensor agrees with the tiled one.
"""

import numpy as np
import pytest
import torch

from oracle.fp8 import E4M3_MAX, dequantize, dequantize_tiles, e4m3_decode, e4m3_encode, quantize_maps, quantize_tiles


def _torch_codes(y):
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("seed", range(4))
def test_encode_matches_torch_cast(seed):
    rng = np.random.default_rng(500 + seed)
    y = np.concatenate([rng.standard_normal(20000) * 10 ** rng.uniform(-4, 2.5, 20000),
                        rng.uniform(-448, 448, 5000), rng.uniform(-2.0 ** -6, 2.0 ** -6, 5000)]).astype(np.float32)
    y = y[np.abs(y) <= 448]                      # the encoder's domain (torch's cast does not saturate)
    assert np.array_equal(e4m3_encode(y), _torch_codes(y))
    big = np.array([449.0, 463.9, 464.0, 1e4, -500.0], np.float32)
    assert e4m3_encode(big).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]   # saturation


def test_ties_and_edges_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[(codes & 0x7F) != 0x7F]
    vals = e4m3_decode(finite)
    # midpoints between neighbouring positive codes (ties go to the even code)
    pos = np.sort(vals[vals >= 0])
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    y = np.concatenate([mids, -mids, vals.astype(np.float32), [0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10]])
    y = y.astype(np.float32)
    assert np.array_equal(e4m3_encode(y), _torch_codes(y))


def test_decode_inverts_encode_on_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes).astype(np.float32)), codes)
    assert e4m3_decode(np.uint8(0x7E)) == 448.0 and e4m3_decode(np.uint8(0x08)) == 2.0 ** -6
    assert e4m3_decode(np.uint8(0x01)) == 2.0 ** -9 and e4m3_decode(np.uint8(0x38)) == 1.0


def test_quantize_maps_scale_and_amax():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((5, 40, 16)) * np.array([1, 3, 0.01, 100, 0])[:, None, None]).astype(np.float32)
    codes, scale = quantize_maps(x)
    amax = np.abs(x.reshape(5, -1)).max(axis=1)
    assert np.array_equal(scale[:4], (amax[:4] / np.float32(448)).astype(np.float32))
    assert scale[4] == np.float32(1.0 / 448)                    # an all-zero map
    for m in range(4):
        i = np.abs(x[m]).argmax()
        assert np.abs(e4m3_decode(codes[m].reshape(-1)[i])) == E4M3_MAX
    deq = dequantize(codes, scale)
    rel = np.abs(deq[:4] - x[:4]) / np.maximum(np.abs(x[:4]), amax[:4, None, None] * 2.0 ** -9 / 448)
    assert rel.max() <= 2.0 ** -4 + 1e-6          # half a unit of 3 mantissa bits (or of the subnormal step)


def test_quantize_tiles_groups_are_independent():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2, 3, 150, 16)).astype(np.float32)   # tiles of 64, 64 and a ragged 22
    x[1, 2, 70] = 500.0                                             # a spike only moves tile 1 of map (1, 2)
    codes, scale = quantize_tiles(x)
    assert codes.shape == x.shape and scale.shape == (2, 3, 3)
    for b, h, j in [(0, 0, 0), (1, 2, 1), (1, 2, 2), (0, 1, 2)]:
        part = x[b, h, 64 * j: 64 * (j + 1)]
        assert scale[b, h, j] == np.float32(np.abs(part).max() / np.float32(448))
        c, s = quantize_maps(part[None])
        assert np.array_equal(codes[b, h, 64 * j: 64 * (j + 1)], c[0]) and s[0] == scale[b, h, j]
    y = x.copy()
    y[1, 2, 70] = 0.0
    c2, s2 = quantize_tiles(y)
    assert np.array_equal(c2[:, :, :64], codes[:, :, :64]) and np.array_equal(c2[:, :, 128:], codes[:, :, 128:])
    assert s2[1, 2, 1] < scale[1, 2, 1]
    # rounding error: half a unit of the 3 mantissa bits for normal codes, half the
    # subnormal step 2^-9 * scale below 2^-6 * scale
    deq = dequantize_tiles(codes, scale)
    sc = np.repeat(scale, 64, axis=2)[:, :, :150, None].astype(np.float64)
    assert np.all(np.abs(deq - x) <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * sc) * (1 + 1e-6))
    assert np.count_nonzero(np.abs(x[1, 2, 64:128]) < 2.0 ** -6 * sc[1, 2, 64:128]) > 0   # subnormals are exercised
