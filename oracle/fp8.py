"""FP8 (e4m3) quantisation of queries and keys (oracle; test infrastructure only).

"LiteVAR: Compressing Visual Autoregressive Modelling with Efficient Attention
and Quantization" (record): the data precision of a VAR model is redundant
and low-bit quantisation keeps its quality.  The record names no format; the
reading taken is 8-bit floating point e4m3 (the OCP "E4M3FN" layout: 1 sign
bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, largest
finite value 448, no infinities) for the attention's queries and keys, with
one scale per group of values (quantize_maps: one group per leading index;
quantize_tiles: one group per (batch, head, 64-token tile)):

    amax  = max |x| over the group (0 -> 1)
    inv   = 448 / amax            (float32, correctly rounded)
    code  = e4m3(x * inv)         (the product in float32; round to nearest even)
    scale = amax / 448            (float32; dequantised value = e4m3 value * scale)

Attention on quantised inputs is then ordinary attention of the dequantised
values, which the attention oracle computes exactly.
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_encode(y):
    """float32 array -> uint8 e4m3 codes, round to nearest even, |y| <= 464 expected.

    Values beyond the largest finite one saturate to +-448 (inputs scaled by
    448/amax never get there beyond rounding).
    """
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    sign = (np.signbit(y)).astype(np.uint8) << 7
    a = np.abs(y)
    out = np.zeros(a.shape, dtype=np.uint8)
    # subnormals: multiples of 2^-9 below 2^-6
    sub = a < 2.0 ** -6
    m = np.rint(a[sub] / 2.0 ** -9)              # rint: round half to even
    out[sub] = m.astype(np.uint8)                # m == 8 is the smallest normal (exponent field 1)
    # normals
    nrm = ~sub
    an = a[nrm]
    e = np.floor(np.log2(an)).astype(np.int64)
    # guard against log2 rounding at exact powers of two
    e = np.where(an < 2.0 ** e, e - 1, e)
    e = np.where(an >= 2.0 ** (e + 1), e + 1, e)
    frac = an / 2.0 ** e - 1.0                   # [0, 1)
    m3 = np.rint(frac * 8.0).astype(np.int64)    # round half to even
    carry = m3 == 8
    e = np.where(carry, e + 1, e)
    m3 = np.where(carry, 0, m3)
    code = (e + 7) * 8 + m3
    code = np.minimum(code, 0x7E)                # saturate at 448
    out[nrm] = code.astype(np.uint8)
    return out | sign


def e4m3_decode(code):
    """uint8 e4m3 codes -> float64 values (0x7F / 0xFF, the NaN codes, are not produced)."""
    code = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 0xF
    m = code & 7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return s * val


def quantize_maps(x):
    """x [maps, ...] (any float dtype) -> (codes uint8 same shape, scale float32 [maps])."""
    x = np.asarray(x, dtype=np.float32)
    maps = x.shape[0]
    flat = x.reshape(maps, -1)
    amax = np.abs(flat).max(axis=1).astype(np.float32)
    amax = np.where(amax > 0, amax, np.float32(1.0)).astype(np.float32)
    inv = (np.float32(E4M3_MAX) / amax).astype(np.float32)
    y = (flat * inv[:, None]).astype(np.float32)
    codes = e4m3_encode(y).reshape(x.shape)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return codes, scale


def dequantize(codes, scale):
    """Dequantised float64 values: e4m3 value * scale of the map (leading axis)."""
    codes = np.asarray(codes)
    v = e4m3_decode(codes)
    return v * np.asarray(scale, dtype=np.float64).reshape((-1,) + (1,) * (codes.ndim - 1))


def quantize_tiles(x, tile=64):
    """x [B, H, T, D] -> (codes uint8 [B, H, T, D], scale float32 [B, H, ceil(T / tile)]).

    Tokens [tile*j, tile*(j+1)) of each (batch, head) form group j (the last
    one may be shorter); each group is quantised as quantize_maps does a map.
    """
    x = np.asarray(x, dtype=np.float32)
    B, H, T, D = x.shape
    n = -(-T // tile)
    codes = np.zeros(x.shape, dtype=np.uint8)
    scale = np.zeros((B, H, n), dtype=np.float32)
    for j in range(n):
        part = x[:, :, tile * j: tile * (j + 1)]
        c, s = quantize_maps(part.reshape((B * H,) + part.shape[2:]))
        codes[:, :, tile * j: tile * (j + 1)] = c.reshape(part.shape)
        scale[:, :, j] = s.reshape(B, H)
    return codes, scale


def dequantize_tiles(codes, scale, tile=64):
    """Dequantised float64 values of quantize_tiles output."""
    v = e4m3_decode(codes)
    T = codes.shape[2]
    s = np.repeat(np.asarray(scale, dtype=np.float64), tile, axis=2)[:, :, :T]
    return v * s[..., None]
