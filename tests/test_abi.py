"""The C ABI on the CPU: the library loads, exports exactly the declared
symbols, and rejects bad arguments on the host before any HIP call (every
case below fails validation, so no device is touched)."""

import ctypes
import os
import re
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "var_attn.h")


@pytest.fixture(scope="module")
def api():
    from scale_wise_attention_amd import api as _api
    return _api


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:var_status|const char\*)\s+(var_\w+)\s*\(", text, flags=re.M)))


def test_exports_match_header(api):
    declared = _declared()
    assert len(declared) == 24
    for name in declared:
        assert hasattr(api.LIB, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True, text=True).stdout
    exported = sorted(ln.split()[-1] for ln in nm.splitlines() if " T " in ln and ln.split()[-1].startswith("var_"))
    assert exported == declared
    assert sorted(api.EXPORTED) == declared


def test_status_strings(api):
    for code, name in api.STATUS.items():
        assert api.LIB.var_status_string(code).decode() == name
    assert api.LIB.var_status_string(99).decode() == "VAR_ERR_UNKNOWN"


W1024 = [1, 2, 4, 6, 8, 12, 16, 20, 24, 32, 40, 48, 64]


def test_extent_and_mask_dims(api):
    assert api.var_schedule_extent((W1024, W1024), 12, 13) == (6425, 4096, 10521)
    assert api.var_schedule_extent((W1024, W1024), 0, 13) == (0, 10521, 10521)
    assert api.var_schedule_extent(([1, 2, 3, 4], [1, 2, 3, 4]), 1, 3) == (1, 13, 14)
    assert api.var_tile_mask_dims((W1024, W1024), 12, 13, api.mask_params()) == (64, 165)
    assert api.var_tile_mask_dims((W1024, W1024), 12, 13, api.mask_params(), n_sel=1638) == (26, 165)
    assert api.var_tile_mask_dims(([1, 2, 3, 4], [1, 2, 3, 4]), 0, 4, api.mask_params(4, 4, 1, 1, 0, 0)) == (8, 8)


FAKE = 1 << 20   # aligned non-null stand-in for a device pointer; never dereferenced


def _dense(api, sched, desc, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, q_index=None, n_sel=0, layout=None):
    L = layout or api.Layout(2 * 16 * 4096 * 128, 4096 * 128, 128)
    P = ctypes.c_void_p
    return api.LIB.var_attn_dense(ctypes.byref(sched) if sched is not None else None,
                                  ctypes.byref(desc) if desc is not None else None,
                                  P(q), L, P(k), L, P(v), L, P(o), L, P(lse), P(q_index), n_sel, P(0))


def _desc(api, **kw):
    d = dict(batch=2, heads=16, head_dim=128, q_scale_begin=12, q_scale_end=13, softmax_scale=0.0,
             in_dtype=api.VAR_BF16, out_dtype=api.VAR_F32)
    d.update(kw)
    return api.AttnDesc(**d)


def _code(api, name):
    return {v: k for k, v in api.STATUS.items()}[name]


def test_dense_validation_errors(api):
    s = api.make_schedule(W1024, W1024)
    E = lambda n: _code(api, n)
    assert _dense(api, None, _desc(api)) == E("VAR_ERR_NULL")
    assert _dense(api, s, None) == E("VAR_ERR_NULL")
    assert _dense(api, api.make_schedule([], []), _desc(api)) == E("VAR_ERR_SCHEDULE")
    assert _dense(api, api.make_schedule([0], [4]), _desc(api, q_scale_begin=0, q_scale_end=1)) == E("VAR_ERR_SCHEDULE")
    assert _dense(api, api.make_schedule([4097], [4]), _desc(api, q_scale_begin=0, q_scale_end=1)) == E("VAR_ERR_SCHEDULE")
    assert _dense(api, api.make_schedule([1] * 33, [1] * 33), _desc(api, q_scale_begin=0, q_scale_end=1)) == E("VAR_ERR_SCHEDULE")
    assert _dense(api, s, _desc(api, q_scale_begin=12, q_scale_end=14)) == E("VAR_ERR_RANGE")
    assert _dense(api, s, _desc(api, q_scale_begin=5, q_scale_end=5)) == E("VAR_ERR_RANGE")
    assert _dense(api, s, _desc(api, batch=0)) == E("VAR_ERR_RANGE")
    assert _dense(api, s, _desc(api, head_dim=96)) == E("VAR_ERR_UNSUPPORTED")
    assert _dense(api, s, _desc(api, head_dim=128, in_dtype=api.VAR_F32)) == E("VAR_ERR_UNSUPPORTED")
    assert _dense(api, s, _desc(api, head_dim=64, in_dtype=api.VAR_F32, out_dtype=api.VAR_BF16)) == E("VAR_ERR_UNSUPPORTED")
    assert _dense(api, s, _desc(api, in_dtype=7)) == E("VAR_ERR_UNSUPPORTED")
    assert _dense(api, s, _desc(api, softmax_scale=-1.0)) == E("VAR_ERR_RANGE")
    assert _dense(api, s, _desc(api, softmax_scale=float("nan"))) == E("VAR_ERR_RANGE")
    assert _dense(api, s, _desc(api), q=0) == E("VAR_ERR_NULL")
    assert _dense(api, s, _desc(api), o=0) == E("VAR_ERR_NULL")
    assert _dense(api, s, _desc(api), k=FAKE + 8) == E("VAR_ERR_STRIDE")
    assert _dense(api, s, _desc(api), layout=api.Layout(0, 0, 100)) == E("VAR_ERR_STRIDE")
    assert _dense(api, s, _desc(api), layout=api.Layout(0, 0, 132)) == E("VAR_ERR_STRIDE")
    assert _dense(api, s, _desc(api), lse=FAKE + 2) == E("VAR_ERR_STRIDE")
    assert _dense(api, s, _desc(api), n_sel=5) == E("VAR_ERR_INDEX")
    assert _dense(api, s, _desc(api), q_index=FAKE, n_sel=4097) == E("VAR_ERR_INDEX")
    assert _dense(api, s, _desc(api), q_index=FAKE, n_sel=3, o=0) == E("VAR_ERR_NULL")
    assert _dense(api, s, _desc(api), q_index=FAKE, n_sel=-1) == E("VAR_ERR_INDEX")
    assert "n_sel" in api.LIB.var_last_error().decode()


def test_empty_selection_returns_ok_without_launch(api):
    s = api.make_schedule(W1024, W1024)
    assert _dense(api, s, _desc(api), q_index=FAKE, n_sel=0) == 0
    assert api.LIB.var_last_error().decode() == ""
    assert _dense(api, s, _desc(api), q_index=FAKE, n_sel=0, o=0) == 0   # empty output tensor


def test_sparse_and_mask_validation_errors(api):
    s = api.make_schedule(W1024, W1024)
    E = lambda n: _code(api, n)
    L = api.Layout(2 * 16 * 4096 * 128, 4096 * 128, 128)
    P = ctypes.c_void_p
    d = _desc(api)
    r = api.LIB.var_attn_block_sparse(ctypes.byref(s), ctypes.byref(d), P(FAKE), L, P(FAKE), L, P(FAKE), L, P(FAKE), L,
                                      P(0), P(0), 0, P(FAKE), P(FAKE), 32, 64, P(0))
    assert r == E("VAR_ERR_UNSUPPORTED")
    r = api.LIB.var_attn_block_sparse(ctypes.byref(s), ctypes.byref(d), P(FAKE), L, P(FAKE), L, P(FAKE), L, P(FAKE), L,
                                      P(0), P(0), 0, P(0), P(FAKE), 64, 64, P(0))
    assert r == E("VAR_ERR_NULL")
    mp = api.mask_params()
    build = api.LIB.var_build_tile_mask
    assert build(ctypes.byref(s), 12, 13, ctypes.byref(mp), P(0), 0, P(FAKE), P(FAKE), 64 * 165 - 1, P(0)) == E("VAR_ERR_CAPACITY")
    assert build(ctypes.byref(s), 12, 13, None, P(0), 0, P(FAKE), P(FAKE), 64 * 165, P(0)) == E("VAR_ERR_NULL")
    assert build(ctypes.byref(s), 12, 13, ctypes.byref(mp), P(0), 0, P(0), P(FAKE), 64 * 165, P(0)) == E("VAR_ERR_NULL")
    assert build(ctypes.byref(s), 12, 13, ctypes.byref(mp), P(0), 3, P(FAKE), P(FAKE), 64 * 165, P(0)) == E("VAR_ERR_INDEX")
    bad = api.mask_params(0, 64)
    assert build(ctypes.byref(s), 12, 13, ctypes.byref(bad), P(0), 0, P(FAKE), P(FAKE), 10 ** 6, P(0)) == E("VAR_ERR_RANGE")
    bad = api.mask_params(64, 64, 7, 7, -1, 2)
    assert build(ctypes.byref(s), 12, 13, ctypes.byref(bad), P(0), 0, P(FAKE), P(FAKE), 10 ** 6, P(0)) == E("VAR_ERR_RANGE")


def test_scatter_validation_errors(api):
    E = lambda n: _code(api, n)
    P = ctypes.c_void_p
    f = api.LIB.var_scatter_restore
    ok_args = dict(maps=32, row_elems=128, dtype=api.VAR_BF16, base=FAKE, bms=2304 * 128, brs=128, h_in=48, w_in=48,
                   upd=FAKE, ums=1638 * 128, urs=128, q_index=FAKE, n_sel=1638, out=FAKE, oms=4096 * 128, ors=128,
                   h_out=64, w_out=64)

    def call(**kw):
        a = dict(ok_args)
        a.update(kw)
        return f(a["maps"], a["row_elems"], a["dtype"], P(a["base"]), a["bms"], a["brs"], a["h_in"], a["w_in"],
                 P(a["upd"]), a["ums"], a["urs"], P(a["q_index"]), a["n_sel"], P(a["out"]), a["oms"], a["ors"],
                 a["h_out"], a["w_out"], P(0), P(0))

    assert call(dtype=5) == E("VAR_ERR_UNSUPPORTED")
    assert call(row_elems=0) == E("VAR_ERR_RANGE")
    assert call(h_out=0) == E("VAR_ERR_RANGE")
    assert call(n_sel=4097) == E("VAR_ERR_INDEX")
    assert call(base=0) == E("VAR_ERR_NULL")
    assert call(q_index=0) == E("VAR_ERR_NULL")
    assert call(brs=64) == E("VAR_ERR_STRIDE")
    assert call(oms=-1) == E("VAR_ERR_STRIDE")
    assert call(maps=0) == 0   # nothing to do, nothing launched


def test_saliency_and_select_validation_errors(api):
    s = api.make_schedule(W1024, W1024)
    E = lambda n: _code(api, n)
    P = ctypes.c_void_p
    L = api.Layout(2 * 16 * 1024 * 128, 1024 * 128, 128)
    sal = api.LIB.var_attn_saliency

    def call(desc, q=FAKE, k=FAKE, lse=FAKE, out=FAKE):
        return sal(ctypes.byref(s), ctypes.byref(desc), P(q), L, P(k), L, P(lse), P(out), P(0))

    assert call(_desc(api, q_scale_begin=9, q_scale_end=11)) == E("VAR_ERR_RANGE")
    assert call(_desc(api, q_scale_begin=9, q_scale_end=10, in_dtype=api.VAR_F32, head_dim=64)) == E("VAR_ERR_UNSUPPORTED")
    assert call(_desc(api, q_scale_begin=9, q_scale_end=10, head_dim=96)) == E("VAR_ERR_UNSUPPORTED")
    assert call(_desc(api, q_scale_begin=9, q_scale_end=10), lse=0) == E("VAR_ERR_NULL")
    assert call(_desc(api, q_scale_begin=9, q_scale_end=10), out=FAKE + 2) == E("VAR_ERR_STRIDE")
    assert call(_desc(api, q_scale_begin=9, q_scale_end=10), q=FAKE + 8) == E("VAR_ERR_STRIDE")
    assert call(_desc(api, q_scale_begin=9, q_scale_end=10, batch=0)) == E("VAR_ERR_RANGE")
    sel = api.LIB.var_select_topk
    assert sel(32, P(FAKE), 32, 32, 64, 64, 4097, P(FAKE), P(0)) == E("VAR_ERR_RANGE")
    assert sel(32, P(FAKE), 32, 32, 64, 64, -1, P(FAKE), P(0)) == E("VAR_ERR_RANGE")
    assert sel(0, P(FAKE), 32, 32, 64, 64, 10, P(FAKE), P(0)) == E("VAR_ERR_RANGE")
    assert sel(32, P(FAKE), 0, 32, 64, 64, 10, P(FAKE), P(0)) == E("VAR_ERR_RANGE")
    assert sel(32, P(FAKE), 91, 91, 128, 128, 10, P(FAKE), P(0)) == E("VAR_ERR_UNSUPPORTED")
    assert sel(32, P(0), 32, 32, 64, 64, 10, P(FAKE), P(0)) == E("VAR_ERR_NULL")
    assert sel(32, P(FAKE), 32, 32, 64, 64, 10, P(FAKE + 2), P(0)) == E("VAR_ERR_STRIDE")
    assert sel(32, P(0), 32, 32, 64, 64, 0, P(0), P(0)) == 0   # nothing to select, nothing launched


def test_split_validation_and_plan(api):
    s = api.make_schedule(W1024, W1024)
    E = lambda n: _code(api, n)
    P = ctypes.c_void_p
    L = api.Layout(2 * 16 * 4096 * 128, 4096 * 128, 128)
    f = api.LIB.var_attn_dense_split

    def call(desc, splits, ws=FAKE, nbytes=1 << 40):
        return f(ctypes.byref(s), ctypes.byref(desc), P(FAKE), L, P(FAKE), L, P(FAKE), L, P(FAKE), L, P(0), P(0), 0,
                 splits, P(ws), nbytes, P(0))

    d = _desc(api)
    assert call(d, 0) == E("VAR_ERR_RANGE")
    assert call(d, 9) == E("VAR_ERR_RANGE")
    assert call(d, 2, ws=0) == E("VAR_ERR_NULL")
    assert call(d, 2, ws=FAKE + 4) == E("VAR_ERR_STRIDE")
    # the 48x48 step: 288 work items of 256 rows; on 256 compute units (the count the
    # library assumes without a device) items 256..287 run split: rows from
    # (b, h) = 28, row 1024 on, 8192 of them, fp32 O and LSE for each of 2 parts
    d48 = _desc(api, q_scale_begin=11, q_scale_end=12)
    need = 2 * (32 * 2304 - (28 * 2304 + 4 * 256)) * 129 * 4
    assert need == 2 * 8192 * 129 * 4
    assert call(d48, 2, nbytes=need - 1) == E("VAR_ERR_CAPACITY")
    f32 = _desc(api, head_dim=64, in_dtype=api.VAR_F32)
    assert call(f32, 2) == E("VAR_ERR_UNSUPPORTED")
    n, nbytes = api.var_attn_split_plan((W1024, W1024), 12, 13, 2, 16, 128)
    assert n == 1 and nbytes == 0                      # 512 work items already fill 256 compute units
    # the 32x32 step: 256 work items of 128 rows fill the 256 compute units; with
    # one batch, 128 items of 40 key tiles leave half of them idle, and their
    # split rows are all of the call's
    assert api.var_attn_split_plan((W1024, W1024), 9, 10, 2, 16, 128) == (1, 0)
    n, nbytes = api.var_attn_split_plan((W1024, W1024), 9, 10, 1, 16, 128)
    assert n > 1 and nbytes == n * 16 * 1024 * 129 * 4
    assert api.var_attn_split_plan((W1024, W1024), 9, 10, 2, 16, 64, dtype=torch.float32) == (1, 0)
    # 288 work items: one whole round of 256 plus 32 items of 101 key tiles that the split spreads
    n, nbytes = api.var_attn_split_plan((W1024, W1024), 11, 12, 2, 16, 128)
    assert n >= 4 and nbytes == n * 8192 * 129 * 4         # only the 32 split items' rows
    # the plan on every 1024px step (256 compute units): dense, then sparse with the
    # mean kept tiles per mask row as the hint; the fewest splits within 3% of the
    # lowest modelled cost (48x48 sparse: 5 splits cost 38.8 units, 4 cost 39.7).
    # Dense steps up to 32x32 run 128-row work items, all in one round: unsplit.
    dense = [api.var_attn_split_plan((W1024, W1024), st, st + 1, 2, 16, 128)[0] for st in range(13)]
    assert dense == [1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 6, 1]
    hints = {7: 11, 8: 15, 9: 18, 10: 21, 11: 25}
    sparse = [api.var_attn_split_plan((W1024, W1024), st, st + 1, 2, 16, 128, kv_tiles_hint=h)[0]
              for st, h in hints.items()]
    assert sparse == [1, 1, 1, 1, 4]
    sp = api.LIB.var_attn_block_sparse_split
    r = sp(ctypes.byref(s), ctypes.byref(d), P(FAKE), L, P(FAKE), L, P(FAKE), L, P(FAKE), L, P(0), P(0), 0,
           P(FAKE), P(FAKE), 64, 64, 9, P(FAKE), 1 << 40, P(0))
    assert r == E("VAR_ERR_RANGE")


def test_decision_scale_validation_errors(api):
    s = api.make_schedule(W1024, W1024)
    E = lambda n: _code(api, n)
    P = ctypes.c_void_p
    L = api.Layout(2 * 16 * 1024 * 128, 1024 * 128, 128)
    bm = api.LIB.var_attn_block_mass
    assert bm(ctypes.byref(s), ctypes.byref(_desc(api, q_scale_begin=9, q_scale_end=11)), P(FAKE), L, P(FAKE), L,
              P(FAKE), P(FAKE), P(0)) == E("VAR_ERR_RANGE")
    big = api.make_schedule([1, 100], [1, 100])       # 10000 rows > 8192
    assert bm(ctypes.byref(big), ctypes.byref(_desc(api, q_scale_begin=1, q_scale_end=2)), P(FAKE), L, P(FAKE), L,
              P(FAKE), P(FAKE), P(0)) == E("VAR_ERR_UNSUPPORTED")
    assert bm(ctypes.byref(s), ctypes.byref(_desc(api, q_scale_begin=9, q_scale_end=10)), P(FAKE), L, P(FAKE), L,
              P(0), P(FAKE), P(0)) == E("VAR_ERR_NULL")
    dt = api.LIB.var_decision_tiles
    assert dt(32, 16, 40, P(FAKE), ctypes.c_float(1.5), P(FAKE), P(0)) == E("VAR_ERR_RANGE")
    assert dt(32, 16, 1025, P(FAKE), ctypes.c_float(0.5), P(FAKE), P(0)) == E("VAR_ERR_UNSUPPORTED")
    assert dt(0, 16, 40, P(FAKE), ctypes.c_float(0.5), P(FAKE), P(0)) == E("VAR_ERR_RANGE")
    assert dt(32, 16, 40, P(0), ctypes.c_float(0.5), P(FAKE), P(0)) == E("VAR_ERR_NULL")
    mm = api.LIB.var_mapped_tile_mask
    assert mm(ctypes.byref(s), 10, 9, 32, P(FAKE), P(FAKE), P(FAKE), 64 * 165, P(0)) == E("VAR_ERR_RANGE")
    assert mm(ctypes.byref(s), 9, 12, 32, P(FAKE), P(FAKE), P(FAKE), 64 * 165 - 1, P(0)) == E("VAR_ERR_CAPACITY")
    assert mm(ctypes.byref(s), 9, 12, 32, P(0), P(FAKE), P(FAKE), 64 * 165, P(0)) == E("VAR_ERR_NULL")
    sh = api.LIB.var_attn_block_sparse_heads
    L2 = api.Layout(2 * 16 * 4096 * 128, 4096 * 128, 128)
    assert sh(ctypes.byref(s), ctypes.byref(_desc(api)), P(FAKE), L2, P(FAKE), L2, P(FAKE), L2, P(FAKE), L2, P(0), P(0),
              0, P(FAKE), P(FAKE), 64 * 165 - 1, P(0)) == E("VAR_ERR_CAPACITY")
    assert sh(ctypes.byref(s), ctypes.byref(_desc(api)), P(FAKE), L2, P(FAKE), L2, P(FAKE), L2, P(FAKE), L2, P(0), P(0),
              0, P(FAKE), P(FAKE), -1, P(0)) == E("VAR_ERR_RANGE")


def test_e4m3_validation_errors(api):
    s = api.make_schedule(W1024, W1024)
    E = lambda n: _code(api, n)
    P = ctypes.c_void_p
    L = api.Layout(2 * 16 * 10521 * 128, 10521 * 128, 128)
    NT = 165                       # 64-token tiles of 10521 keys
    qz = api.LIB.var_quantize_e4m3

    def quant(b=2, h=16, t=10521, d=128, x=FAKE, xl=L, c=FAKE, cl=L, sc=FAKE, stride=NT, first=0):
        return qz(b, h, t, d, P(x), xl, P(c), cl, P(sc), stride, first, P(0))

    assert quant(h=0) == E("VAR_ERR_RANGE")
    assert quant(b=256, h=256) == E("VAR_ERR_RANGE")                 # > 65535 maps
    assert quant(first=10522) == E("VAR_ERR_RANGE")
    assert quant(first=-1) == E("VAR_ERR_RANGE")
    assert quant(d=120) == E("VAR_ERR_UNSUPPORTED")
    assert quant(d=512) == E("VAR_ERR_UNSUPPORTED")
    assert quant(sc=0) == E("VAR_ERR_NULL")
    assert quant(x=FAKE + 8) == E("VAR_ERR_STRIDE")
    assert quant(stride=NT - 1) == E("VAR_ERR_STRIDE")
    odd = api.Layout(2 * 16 * 10521 * 136, 10521 * 136, 136)   # 136-byte code rows: not a multiple of 16
    assert quant(cl=odd) == E("VAR_ERR_STRIDE")
    assert quant(first=10521, x=0, c=0, sc=0) == E("VAR_OK")     # no tile to write: nothing is touched
    dn = api.LIB.var_attn_dense_e4m3
    Lq = api.Layout(2 * 16 * 4096 * 128, 4096 * 128, 128)

    def dense(desc, ks=FAKE, kl=L, kst=NT):
        return dn(ctypes.byref(s), ctypes.byref(desc), P(FAKE), Lq, P(FAKE), kl, P(ks), kst, P(FAKE), L,
                  P(FAKE), Lq, P(0), P(0), 0, 1, P(0), 0, P(0))

    assert dense(_desc(api, head_dim=64)) == E("VAR_ERR_UNSUPPORTED")
    assert dense(_desc(api, in_dtype=api.VAR_F32, head_dim=64)) == E("VAR_ERR_UNSUPPORTED")
    assert dense(_desc(api), ks=0) == E("VAR_ERR_NULL")
    assert dense(_desc(api), ks=FAKE + 2) == E("VAR_ERR_STRIDE")
    assert dense(_desc(api), kl=odd) == E("VAR_ERR_STRIDE")
    assert dense(_desc(api), kst=NT - 1) == E("VAR_ERR_STRIDE")
    sp = api.LIB.var_attn_block_sparse_e4m3

    def sparse(rp=FAKE, stride=0):
        return sp(ctypes.byref(s), ctypes.byref(_desc(api)), P(FAKE), Lq, P(FAKE), L, P(FAKE), NT,
                  P(FAKE), L, P(FAKE), Lq, P(0), P(0), 0, P(rp), P(FAKE), stride, P(0))

    assert sparse(stride=-1) == E("VAR_ERR_RANGE")
    assert sparse(stride=64 * 165 - 1) == E("VAR_ERR_CAPACITY")
    assert sparse(rp=0) == E("VAR_ERR_NULL")


def test_out_at_index_needs_q_index(api):
    """out_at_index = 1 without a q_index, or another value, is rejected before any HIP call."""
    s = api.make_schedule(W1024, W1024)
    assert _dense(api, s, _desc(api, out_at_index=1)) == _code(api, "VAR_ERR_INDEX")
    assert _dense(api, s, _desc(api, out_at_index=2), q_index=FAKE, n_sel=16) == _code(api, "VAR_ERR_RANGE")


def test_restore_validation_errors(api):
    """var_attn_block_sparse_restore refuses, before any HIP call, what its one
    launch cannot do: more than one step, fp32 input, out_at_index other than 1,
    misaligned or non-uniform map strides, and bad selections."""
    s = api.make_schedule(W1024, W1024)
    E = lambda n: _code(api, n)
    P = ctypes.c_void_p
    L = api.Layout(16 * 4096 * 128, 4096 * 128, 128)
    LB = api.Layout(16 * 2304 * 128, 2304 * 128, 128)

    def call(desc=None, base=FAKE, base_l=None, o_l=None, q_index=FAKE, n_sel=1638, h_in=48, w_in=48):
        d = desc or _desc(api, out_at_index=1, out_dtype=api.VAR_BF16)
        return api.LIB.var_attn_block_sparse_restore(
            ctypes.byref(s), ctypes.byref(d), P(FAKE), L, P(FAKE), L, P(FAKE), L, P(FAKE), o_l or L, P(0),
            P(q_index), n_sel, P(FAKE), P(FAKE), 64, 64, P(base), base_l or LB, h_in, w_in, P(0), P(0))

    assert call(desc=_desc(api, out_at_index=1, q_scale_begin=11)) == E("VAR_ERR_RANGE")
    assert call(desc=_desc(api, out_at_index=0)) == E("VAR_ERR_RANGE")
    assert call(desc=_desc(api, out_at_index=1, head_dim=64, in_dtype=api.VAR_F32)) == E("VAR_ERR_UNSUPPORTED")
    assert call(desc=_desc(api, out_at_index=1, head_dim=96)) == E("VAR_ERR_UNSUPPORTED")
    assert call(base=0) == E("VAR_ERR_NULL")
    assert call(base=FAKE + 8) == E("VAR_ERR_STRIDE")
    assert call(base_l=api.Layout(16 * 2304 * 132, 2304 * 132, 132)) == E("VAR_ERR_STRIDE")
    assert call(base_l=api.Layout(2304 * 128, 2304 * 128, 128)) == E("VAR_ERR_STRIDE")
    assert call(o_l=api.Layout(0, 4096 * 128, 128)) == E("VAR_ERR_STRIDE")
    assert call(h_in=0) == E("VAR_ERR_RANGE")
    assert call(n_sel=4097) == E("VAR_ERR_INDEX")
    assert call(n_sel=-1) == E("VAR_ERR_INDEX")
    assert call(q_index=0) == E("VAR_ERR_NULL")
    assert "q_index" in api.LIB.var_last_error().decode()


def test_device_info_without_a_device(api):
    """No HIP device here: the query reports VAR_ERR_HIP instead of a made-up count."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present (the GPU tests check the values)")
    with pytest.raises(api.VarAttnError) as e:
        api.var_device_info()
    assert e.value.status_name == "VAR_ERR_HIP"


def test_noalloc_split_rejects_oversized_calls_before_any_hip_call(api):
    """The allocation-free split call checks its partials against the static scratch
    first: 8 parts of the 24x24 step (160 work items of 128 rows, all split: 76 MB)
    exceed the 64 MiB."""
    s = api.make_schedule(W1024, W1024)
    L = api.Layout(2 * 16 * 4096 * 128, 4096 * 128, 128)
    P = ctypes.c_void_p
    d = _desc(api, q_scale_begin=8, q_scale_end=9)
    r = api.LIB.var_attn_dense_split_noalloc(ctypes.byref(s), ctypes.byref(d), P(FAKE), L, P(FAKE), L, P(FAKE), L,
                                             P(FAKE), L, P(0), P(0), 0, 8, P(0))
    assert r == _code(api, "VAR_ERR_CAPACITY")
    assert b"static scratch" in api.LIB.var_last_error()
    assert api.LIB.var_attn_dense_split_noalloc(ctypes.byref(s), ctypes.byref(d), P(FAKE), L, P(FAKE), L, P(FAKE),
                                                L, P(FAKE), L, P(0), P(0), 0, 9, P(0)) == _code(api, "VAR_ERR_RANGE")


def test_batched_masks_validation_errors(api):
    """var_build_tile_masks checks every call on the host before it launches anything,
    and names the call that failed."""
    s = api.make_schedule(W1024, W1024)
    mp = api.mask_params()
    P = ctypes.c_void_p
    build = api.LIB.var_build_tile_masks

    def calls(*cs):
        arr = (api.TileMaskCall * len(cs))()
        for i, c in enumerate(cs):
            arr[i] = api.TileMaskCall(*c)
        return arr

    good = (12, 13, None, 0, FAKE, FAKE, 64 * 165)
    assert build(ctypes.byref(s), ctypes.byref(mp), None, 1, P(0)) == _code(api, "VAR_ERR_NULL")
    assert build(ctypes.byref(s), ctypes.byref(mp), calls(good), 0, P(0)) == _code(api, "VAR_ERR_RANGE")
    many = calls(*([good] * (api.MAX_MASK_CALLS + 1)))
    assert build(ctypes.byref(s), ctypes.byref(mp), many, api.MAX_MASK_CALLS + 1, P(0)) == _code(api, "VAR_ERR_RANGE")
    # call 1: a scale range past the schedule
    r = build(ctypes.byref(s), ctypes.byref(mp), calls(good, (12, 14, None, 0, FAKE, FAKE, 64 * 165)), 2, P(0))
    assert r == _code(api, "VAR_ERR_RANGE") and api.LIB.var_last_error().startswith(b"call 1: ")
    # call 2: col_idx too small for its 26 x 165 pruned mask
    short = (12, 13, FAKE, 1638, FAKE, FAKE, 26 * 165 - 1)
    r = build(ctypes.byref(s), ctypes.byref(mp), calls(good, good, short), 3, P(0))
    assert r == _code(api, "VAR_ERR_CAPACITY") and b"call 2" in api.LIB.var_last_error()
    # call 0: NULL row_ptr
    r = build(ctypes.byref(s), ctypes.byref(mp), calls((11, 12, None, 0, None, FAKE, 36 * 101)), 1, P(0))
    assert r == _code(api, "VAR_ERR_NULL") and b"call 0" in api.LIB.var_last_error()
    # the mask rule itself is checked as in var_build_tile_mask
    bad = api.mask_params(0, 64)
    assert build(ctypes.byref(s), ctypes.byref(bad), calls(good), 1, P(0)) == _code(api, "VAR_ERR_RANGE")
