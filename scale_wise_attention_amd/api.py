"""Thin ctypes binding over libvarattn.so (include/var_attn.h).

Argument marshalling only: tensors become device pointers plus element
strides, the schedule becomes two int32 host arrays, the current torch stream
becomes the hipStream_t.  Every computation happens in the library's HIP
kernels; there is no fallback.  Importing this module raises if the library
has not been built (``python -m scale_wise_attention_amd.build``).

Functions carry the C names: ``var_attn_dense``, ``var_build_tile_mask``,
``var_attn_block_sparse``, ``var_scatter_restore``, ``var_attn_saliency``,
``var_select_topk`` (plus the host-only helpers ``var_schedule_extent`` and
``var_tile_mask_dims``).
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvarattn.so")

VAR_F32 = 0
VAR_BF16 = 1

STATUS = {0: "VAR_OK", 1: "VAR_ERR_NULL", 2: "VAR_ERR_SCHEDULE", 3: "VAR_ERR_RANGE",
          4: "VAR_ERR_UNSUPPORTED", 5: "VAR_ERR_STRIDE", 6: "VAR_ERR_CAPACITY",
          7: "VAR_ERR_INDEX", 8: "VAR_ERR_HIP"}
MAX_SCALES = 32

EXPORTED = ("var_schedule_extent", "var_attn_dense", "var_tile_mask_dims", "var_build_tile_mask",
            "var_attn_block_sparse", "var_scatter_restore", "var_attn_saliency", "var_select_topk",
            "var_attn_dense_split", "var_attn_block_sparse_split", "var_attn_split_plan",
            "var_attn_block_mass", "var_decision_tiles", "var_mapped_tile_mask", "var_attn_block_sparse_heads",
            "var_quantize_e4m3", "var_attn_dense_e4m3", "var_attn_block_sparse_e4m3", "var_device_info",
            "var_attn_dense_split_noalloc", "var_build_tile_masks", "var_attn_block_sparse_restore",
            "var_status_string", "var_last_error")


class VarAttnError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        self.status_name = STATUS.get(status, f"status {status}")
        super().__init__(f"{self.status_name}: {detail}")


class Schedule(ctypes.Structure):
    _fields_ = [("num_scales", ctypes.c_int32), ("h", ctypes.POINTER(ctypes.c_int32)),
                ("w", ctypes.POINTER(ctypes.c_int32))]


class Layout(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("token", ctypes.c_int64)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("q_scale_begin", ctypes.c_int32), ("q_scale_end", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("out_at_index", ctypes.c_int32)]


class MaskParams(ctypes.Structure):
    _fields_ = [("tile_q", ctypes.c_int32), ("tile_k", ctypes.c_int32), ("sink_scales", ctypes.c_int32),
                ("local_from_scale", ctypes.c_int32), ("radius_y", ctypes.c_int32), ("radius_x", ctypes.c_int32)]


class TileMaskCall(ctypes.Structure):
    _fields_ = [("q_scale_begin", ctypes.c_int32), ("q_scale_end", ctypes.c_int32), ("q_index", ctypes.c_void_p),
                ("n_sel", ctypes.c_int32), ("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
                ("col_capacity", ctypes.c_int64)]


MAX_MASK_CALLS = 16


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m scale_wise_attention_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    SP = ctypes.POINTER(Schedule)
    lib.var_schedule_extent.argtypes = [SP, i32, i32, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.var_attn_dense.argtypes = [SP, ctypes.POINTER(AttnDesc), P, Layout, P, Layout, P, Layout, P, Layout,
                                   P, P, i32, P]
    lib.var_tile_mask_dims.argtypes = [SP, i32, i32, ctypes.POINTER(MaskParams), i32,
                                       ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.var_build_tile_mask.argtypes = [SP, i32, i32, ctypes.POINTER(MaskParams), P, i32, P, P, i64, P]
    lib.var_build_tile_masks.argtypes = [SP, ctypes.POINTER(MaskParams), ctypes.POINTER(TileMaskCall), i32, P]
    lib.var_attn_block_sparse.argtypes = [SP, ctypes.POINTER(AttnDesc), P, Layout, P, Layout, P, Layout, P, Layout,
                                          P, P, i32, P, P, i32, i32, P]
    lib.var_attn_block_sparse_restore.argtypes = [SP, ctypes.POINTER(AttnDesc), P, Layout, P, Layout, P, Layout, P,
                                                  Layout, P, P, i32, P, P, i32, i32, P, Layout, i32, i32, P, P]
    lib.var_scatter_restore.argtypes = [i32, i32, ctypes.c_int, P, i64, i64, i32, i32, P, i64, i64, P, i32,
                                        P, i64, i64, i32, i32, P, P]
    lib.var_attn_saliency.argtypes = [SP, ctypes.POINTER(AttnDesc), P, Layout, P, Layout, P, P, P]
    lib.var_select_topk.argtypes = [i32, P, i32, i32, i32, i32, i32, P, P]
    lib.var_attn_dense_split.argtypes = [SP, ctypes.POINTER(AttnDesc), P, Layout, P, Layout, P, Layout, P, Layout,
                                         P, P, i32, i32, P, i64, P]
    lib.var_attn_block_sparse_split.argtypes = [SP, ctypes.POINTER(AttnDesc), P, Layout, P, Layout, P, Layout, P,
                                                Layout, P, P, i32, P, P, i32, i32, i32, P, i64, P]
    lib.var_attn_split_plan.argtypes = [SP, ctypes.POINTER(AttnDesc), i32, i32, ctypes.POINTER(i32),
                                        ctypes.POINTER(i64)]
    lib.var_attn_block_mass.argtypes = [SP, ctypes.POINTER(AttnDesc), P, Layout, P, Layout, P, P, P]
    lib.var_decision_tiles.argtypes = [i32, i32, i32, P, ctypes.c_float, P, P]
    lib.var_mapped_tile_mask.argtypes = [SP, i32, i32, i32, P, P, P, i64, P]
    lib.var_attn_block_sparse_heads.argtypes = [SP, ctypes.POINTER(AttnDesc), P, Layout, P, Layout, P, Layout, P,
                                                Layout, P, P, i32, P, P, i64, P]
    lib.var_quantize_e4m3.argtypes = [i32, i32, i32, i32, P, Layout, P, Layout, P, i64, i32, P]
    lib.var_attn_dense_e4m3.argtypes = [SP, ctypes.POINTER(AttnDesc), P, Layout, P, Layout, P, i64, P,
                                        Layout, P, Layout, P, P, i32, i32, P, i64, P]
    lib.var_attn_block_sparse_e4m3.argtypes = [SP, ctypes.POINTER(AttnDesc), P, Layout, P, Layout, P, i64,
                                               P, Layout, P, Layout, P, P, i32, P, P, i64, P]
    lib.var_device_info.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.var_attn_dense_split_noalloc.argtypes = [SP, ctypes.POINTER(AttnDesc), P, Layout, P, Layout, P, Layout, P,
                                                 Layout, P, P, i32, i32, P]
    for name in EXPORTED[:-2]:
        getattr(lib, name).restype = ctypes.c_int
    lib.var_status_string.argtypes = [ctypes.c_int]
    lib.var_status_string.restype = ctypes.c_char_p
    lib.var_last_error.argtypes = []
    lib.var_last_error.restype = ctypes.c_char_p
    return lib


LIB = _load()


def _check(status):
    if status != 0:
        raise VarAttnError(status, LIB.var_last_error().decode())


def make_schedule(h, w):
    """ctypes schedule; keeps its host arrays alive on the returned object."""
    h = [int(a) for a in h]
    w = [int(a) for a in w]
    if len(h) != len(w):
        raise ValueError("h and w differ in length")
    ha = (ctypes.c_int32 * max(1, len(h)))(*h)
    wa = (ctypes.c_int32 * max(1, len(w)))(*w)
    s = Schedule(len(h), ctypes.cast(ha, ctypes.POINTER(ctypes.c_int32)), ctypes.cast(wa, ctypes.POINTER(ctypes.c_int32)))
    s._keep = (ha, wa)
    return s


def _as_schedule(schedule):
    if isinstance(schedule, Schedule):
        return schedule
    h, w = schedule
    return make_schedule(h, w)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _layout(t):
    """[B, H, T, D] tensor -> element strides; the last dim must be contiguous."""
    if t.dim() != 4:
        raise ValueError("expected a [batch, head, token, dim] tensor")
    if t.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous (stride 1)")
    return Layout(t.stride(0), t.stride(1), t.stride(2))


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return VAR_BF16
    if dt == torch.float32:
        return VAR_F32
    raise ValueError(f"unsupported dtype {dt}")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def var_schedule_extent(schedule, q_scale_begin, q_scale_end):
    """(first_token, n_q, kv_len) of queries of scales [begin, end)."""
    s = _as_schedule(schedule)
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(LIB.var_schedule_extent(ctypes.byref(s), q_scale_begin, q_scale_end, ctypes.byref(a),
                                   ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def _check_index(q_index, device):
    if q_index is None:
        return
    if q_index.dtype != torch.int32 or q_index.dim() != 1 or not q_index.is_contiguous():
        raise ValueError("q_index must be a contiguous 1-D int32 tensor")
    if q_index.device != device:
        raise ValueError("q_index must live on the tensors' device")


def _attn_common(schedule, q, k, v, q_scale_begin, q_scale_end, out, out_dtype, softmax_scale, q_index, want_lse,
                 qk_codes=False, out_at_index=False):
    s = _as_schedule(schedule)
    _, n_q, kv_len = var_schedule_extent(s, q_scale_begin, q_scale_end)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4 or not t.is_cuda:
            raise ValueError(f"{name} must be a 4-D device tensor [batch, head, token, dim]")
    B, H, _, D = q.shape
    if k.shape[0] != B or v.shape[0] != B or k.shape[1] != H or v.shape[1] != H or k.shape[3] != D or v.shape[3] != D:
        raise ValueError("q, k, v disagree in batch, heads or head_dim")
    if qk_codes:
        if q.dtype != torch.bfloat16 or k.dtype != torch.uint8 or v.dtype != torch.bfloat16:
            raise ValueError("e4m3 attention takes bf16 q and v and uint8 codes for k")
    elif q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share a dtype")
    if q.device != k.device or q.device != v.device:
        raise ValueError("q, k, v must share a device")
    if q.shape[2] < n_q:
        raise ValueError(f"q holds {q.shape[2]} tokens, the scales need {n_q}")
    if k.shape[2] < kv_len or v.shape[2] < kv_len:
        raise ValueError(f"k/v hold fewer than kv_len={kv_len} tokens")
    _check_index(q_index, q.device)
    rows = n_q if q_index is None else int(q_index.numel())
    if out_at_index and q_index is None:
        raise ValueError("out_at_index needs q_index")
    out_rows = n_q if out_at_index else rows      # out_at_index: row i goes to row q_index[i] of the full grid
    if out is None:
        odt = out_dtype if out_dtype is not None else torch.float32
        out = torch.empty((B, H, out_rows, D), dtype=odt, device=q.device)
    elif tuple(out.shape) != (B, H, out_rows, D) or out.device != q.device:
        raise ValueError(f"out must have shape {(B, H, out_rows, D)} on q's device")
    lse = torch.empty((B, H, rows), dtype=torch.float32, device=q.device) if want_lse else None
    desc = AttnDesc(B, H, D, q_scale_begin, q_scale_end, float(softmax_scale), _dtype_code(v.dtype),
                    _dtype_code(out.dtype), 1 if out_at_index else 0)
    return s, desc, out, lse, rows


def var_device_info():
    """(compute units, peak engine clock in kHz) of the current device, as the library reads them."""
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _check(LIB.var_device_info(ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def var_attn_split_plan(schedule, q_scale_begin, q_scale_end, batch, heads, head_dim, n_sel=0, kv_tiles_hint=0,
                        dtype=torch.bfloat16):
    """(n_splits, workspace_bytes) the library picks for a call of this shape."""
    s = _as_schedule(schedule)
    desc = AttnDesc(batch, heads, head_dim, q_scale_begin, q_scale_end, 0.0, _dtype_code(dtype), VAR_F32)
    a, b = ctypes.c_int32(), ctypes.c_int64()
    _check(LIB.var_attn_split_plan(ctypes.byref(s), ctypes.byref(desc), int(n_sel), int(kv_tiles_hint),
                                   ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def split_workspace(n_splits, batch, heads, rows, head_dim, device="cuda"):
    """A workspace tensor for var_attn_*(..., n_splits=n_splits)."""
    n = n_splits * batch * heads * rows * (head_dim + 1) if n_splits > 1 else 0
    return torch.empty(max(1, n), dtype=torch.float32, device=device)


def _ws_args(n_splits, workspace):
    if n_splits == 1 and workspace is None:
        return ctypes.c_void_p(0), 0
    if workspace is None:
        raise ValueError("n_splits > 1 needs a workspace (see split_workspace)")
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def var_attn_dense(schedule, q, k, v, q_scale_begin, q_scale_end, out=None, out_dtype=None,
                   softmax_scale=0.0, q_index=None, return_lse=False, n_splits=1, workspace=None, out_at_index=False):
    """Dense block-causal attention of the queries of scales [begin, end).

    q [B, H, n_q, D] (row j = token off[begin] + j), k / v [B, H, >= kv_len, D];
    returns out [B, H, rows, D] (and lse [B, H, rows]); rows = len(q_index) or n_q.
    n_splits > 1 runs the key-split variant in `workspace`.  out_at_index: output row i is
    written to row q_index[i] of out [B, H, n_q, D] (other rows untouched).
    """
    s, desc, out, lse, rows = _attn_common(schedule, q, k, v, q_scale_begin, q_scale_end, out, out_dtype,
                                           softmax_scale, q_index, return_lse, out_at_index=out_at_index)
    n_sel = rows if q_index is not None else 0
    if q_index is not None and n_sel == 0:   # an empty selection has no device pointer: nothing to compute
        return (out, lse) if return_lse else out
    args = (ctypes.byref(s), ctypes.byref(desc), _ptr(q), _layout(q), _ptr(k), _layout(k), _ptr(v), _layout(v),
            _ptr(out), _layout(out), _ptr(lse), _ptr(q_index), n_sel)
    if n_splits == 1 and workspace is None:
        _check(LIB.var_attn_dense(*args, _stream(q.device)))
    else:
        wp, wb = _ws_args(n_splits, workspace)
        _check(LIB.var_attn_dense_split(*args, int(n_splits), wp, wb, _stream(q.device)))
    return (out, lse) if return_lse else out


def var_attn_dense_split_noalloc(schedule, q, k, v, q_scale_begin, q_scale_end, n_splits, out=None,
                                 out_dtype=None, softmax_scale=0.0, q_index=None, return_lse=False,
                                 out_at_index=False):
    """var_attn_dense with n_splits key splits whose partials go to the library's static
    device scratch instead of a workspace (no allocation in the call)."""
    s, desc, out, lse, rows = _attn_common(schedule, q, k, v, q_scale_begin, q_scale_end, out, out_dtype,
                                           softmax_scale, q_index, return_lse, out_at_index=out_at_index)
    n_sel = rows if q_index is not None else 0
    if q_index is not None and n_sel == 0:
        return (out, lse) if return_lse else out
    _check(LIB.var_attn_dense_split_noalloc(ctypes.byref(s), ctypes.byref(desc), _ptr(q), _layout(q), _ptr(k),
                                            _layout(k), _ptr(v), _layout(v), _ptr(out), _layout(out), _ptr(lse),
                                            _ptr(q_index), n_sel, int(n_splits), _stream(q.device)))
    return (out, lse) if return_lse else out


def var_tile_mask_dims(schedule, q_scale_begin, q_scale_end, mask_params, n_sel=0):
    s = _as_schedule(schedule)
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _check(LIB.var_tile_mask_dims(ctypes.byref(s), q_scale_begin, q_scale_end, ctypes.byref(mask_params), n_sel,
                                  ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def mask_params(tile_q=64, tile_k=64, sink_scales=7, local_from_scale=7, radius_y=2, radius_x=2):
    return MaskParams(tile_q, tile_k, sink_scales, local_from_scale, radius_y, radius_x)


def var_build_tile_mask(schedule, q_scale_begin, q_scale_end, params, q_index=None, device="cuda",
                        row_ptr=None, col_idx=None):
    """Device CSR (row_ptr int32 [n_qt+1], col_idx int32 [n_qt*n_kt] staging buffer)."""
    s = _as_schedule(schedule)
    n_sel = 0 if q_index is None else int(q_index.numel())
    dev = q_index.device if q_index is not None else torch.device(device)
    _check_index(q_index, dev)
    n_qt, n_kt = var_tile_mask_dims(s, q_scale_begin, q_scale_end, params, n_sel)
    if q_index is not None and n_sel == 0:
        n_qt = 0          # empty selection: row_ptr = [0]
    if row_ptr is None:
        row_ptr = torch.empty(n_qt + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(max(1, n_qt * n_kt), dtype=torch.int32, device=dev)
    if row_ptr.numel() < n_qt + 1 or row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise ValueError("row_ptr must be int32 with n_qt+1 entries; col_idx int32")
    qi = _ptr(q_index)
    if q_index is not None and n_sel == 0:
        # an empty tensor has no device pointer; the ABI tells "empty selection" from "no
        # selection" by a non-NULL q_index with n_sel = 0 (never read), so pass row_ptr's address
        qi = _ptr(row_ptr)
    _check(LIB.var_build_tile_mask(ctypes.byref(s), q_scale_begin, q_scale_end, ctypes.byref(params),
                                   qi, n_sel, _ptr(row_ptr), _ptr(col_idx), col_idx.numel(),
                                   _stream(dev)))
    return row_ptr, col_idx


def var_build_tile_masks(schedule, params, calls, device="cuda"):
    """Several tile masks of one schedule and rule in one pair of launches.  calls: a
    list of (q_scale_begin, q_scale_end, q_index or None[, row_ptr, col_idx]); returns the
    list of (row_ptr, col_idx), each as var_build_tile_mask would return it."""
    s = _as_schedule(schedule)
    if not 1 <= len(calls) <= MAX_MASK_CALLS:
        raise ValueError(f"1 to {MAX_MASK_CALLS} calls")
    arr = (TileMaskCall * len(calls))()
    out = []
    dev = torch.device(device)
    for i, c in enumerate(calls):
        b, e, q_index = c[0], c[1], c[2]
        row_ptr, col_idx = (c[3], c[4]) if len(c) > 3 else (None, None)
        n_sel = 0 if q_index is None else int(q_index.numel())
        d = q_index.device if q_index is not None else dev
        _check_index(q_index, d)
        n_qt, n_kt = var_tile_mask_dims(s, b, e, params, n_sel)
        if q_index is not None and n_sel == 0:
            n_qt = 0          # empty selection: row_ptr = [0]
        if row_ptr is None:
            row_ptr = torch.empty(n_qt + 1, dtype=torch.int32, device=d)
        if col_idx is None:
            col_idx = torch.empty(max(1, n_qt * n_kt), dtype=torch.int32, device=d)
        if row_ptr.numel() < n_qt + 1 or row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
            raise ValueError("row_ptr must be int32 with n_qt+1 entries; col_idx int32")
        qi = _ptr(q_index)
        if q_index is not None and n_sel == 0:
            qi = _ptr(row_ptr)     # non-NULL q_index with n_sel = 0: the empty selection (never read)
        arr[i] = TileMaskCall(b, e, qi.value, n_sel, _ptr(row_ptr).value, _ptr(col_idx).value, col_idx.numel())
        out.append((row_ptr, col_idx))
    _check(LIB.var_build_tile_masks(ctypes.byref(s), ctypes.byref(params), arr, len(calls), _stream(dev)))
    return out


def var_attn_block_sparse(schedule, q, k, v, q_scale_begin, q_scale_end, row_ptr, col_idx, out=None,
                          out_dtype=None, softmax_scale=0.0, q_index=None, return_lse=False, tile_q=64, tile_k=64,
                          n_splits=1, workspace=None, out_at_index=False):
    s, desc, out, lse, rows = _attn_common(schedule, q, k, v, q_scale_begin, q_scale_end, out, out_dtype,
                                           softmax_scale, q_index, return_lse, out_at_index=out_at_index)
    n_sel = rows if q_index is not None else 0
    if q_index is not None and n_sel == 0:
        return (out, lse) if return_lse else out
    n_qt = -(-rows // tile_q)
    for name, t in (("row_ptr", row_ptr), ("col_idx", col_idx)):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous 1-D int32 tensor on q's device")
    if row_ptr.numel() < n_qt + 1:
        raise ValueError(f"row_ptr needs {n_qt + 1} entries")
    args = (ctypes.byref(s), ctypes.byref(desc), _ptr(q), _layout(q), _ptr(k), _layout(k), _ptr(v), _layout(v),
            _ptr(out), _layout(out), _ptr(lse), _ptr(q_index), n_sel, _ptr(row_ptr), _ptr(col_idx), tile_q, tile_k)
    if n_splits == 1 and workspace is None:
        _check(LIB.var_attn_block_sparse(*args, _stream(q.device)))
    else:
        wp, wb = _ws_args(n_splits, workspace)
        _check(LIB.var_attn_block_sparse_split(*args, int(n_splits), wp, wb, _stream(q.device)))
    return (out, lse) if return_lse else out


def var_attn_block_sparse_restore(schedule, q, k, v, step, row_ptr, col_idx, q_index, base, h_in, w_in, out=None,
                                  out_dtype=None, softmax_scale=0.0, return_lse=False, err_flag=None, tile_q=64,
                                  tile_k=64):
    """Pruned block-sparse attention of one step plus its reconstruction, in one launch
    (two when the attention leaves fewer than 64 compute-unit slots free).

    Output row i of the attention over the queries q_index (ascending positions of
    the step's grid) goes to row q_index[i] of out [B, H, h*w, D]; every other row
    of out is the nearest-upsampled row of base [B, H, >= h_in*w_in, D].
    """
    s, desc, out, lse, rows = _attn_common(schedule, q, k, v, step, step + 1, out, out_dtype, softmax_scale,
                                           q_index, return_lse, out_at_index=True)
    n_sel = rows
    if base.dim() != 4 or base.dtype != out.dtype or base.device != q.device or base.stride(3) != 1:
        raise ValueError("base must be a [B, H, tokens, D] device tensor of out's dtype with contiguous rows")
    if tuple(base.shape[:2]) != tuple(out.shape[:2]) or base.shape[3] != out.shape[3] or base.shape[2] < h_in * w_in:
        raise ValueError("base must be [B, H, >= h_in*w_in, D] with out's B, H and D")
    n_qt = -(-rows // tile_q)
    for name, t in (("row_ptr", row_ptr), ("col_idx", col_idx)):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous 1-D int32 tensor on q's device")
    if row_ptr.numel() < n_qt + 1:
        raise ValueError(f"row_ptr needs {n_qt + 1} entries")
    _check(LIB.var_attn_block_sparse_restore(
        ctypes.byref(s), ctypes.byref(desc), _ptr(q), _layout(q), _ptr(k), _layout(k), _ptr(v), _layout(v),
        _ptr(out), _layout(out), _ptr(lse), _ptr(q_index), n_sel, _ptr(row_ptr), _ptr(col_idx), tile_q, tile_k,
        _ptr(base), _layout(base), h_in, w_in, _ptr(err_flag), _stream(q.device)))
    return (out, lse) if return_lse else out


def var_scatter_restore(base, h_in, w_in, upd, q_index, h_out, w_out, out=None, err_flag=None):
    """base [M, h_in*w_in, E], upd [M, n_sel, E], q_index int32 [n_sel] -> out [M, h_out*w_out, E].

    Tensors of 4 dims [B, H, T, E] are accepted and treated as M = B*H maps
    (they must then be viewable as [B*H, T, E]).
    """
    def as3(t):
        return t.view(-1, t.shape[-2], t.shape[-1]) if t.dim() == 4 else t

    b3 = as3(base)
    M, _, E = b3.shape
    n_sel = 0 if q_index is None else int(q_index.numel())
    u3 = as3(upd) if (upd is not None and n_sel > 0) else None
    if out is None:
        shape = (*base.shape[:-2], h_out * w_out, E)
        out = torch.empty(shape, dtype=base.dtype, device=base.device)
    o3 = as3(out)
    _check_index(q_index, base.device)
    if b3.shape[1] < h_in * w_in:
        raise ValueError("base holds fewer than h_in*w_in rows")
    if o3.shape[0] != M or o3.shape[2] != E or o3.shape[1] < h_out * w_out or o3.dtype != base.dtype:
        raise ValueError("out must be [maps, >= h_out*w_out, E] of base's dtype")
    if u3 is not None and (u3.shape[0] != M or u3.shape[2] != E or u3.shape[1] < n_sel or u3.dtype != base.dtype):
        raise ValueError("upd must be [maps, >= n_sel, E] of base's dtype")
    for t in (b3, o3) + ((u3,) if u3 is not None else ()):
        if t.stride(2) != 1 or not t.is_cuda or t.device != base.device:
            raise ValueError("rows must be contiguous device tensors on one device")
    _check(LIB.var_scatter_restore(M, E, _dtype_code(base.dtype), _ptr(b3), b3.stride(0), b3.stride(1), h_in, w_in,
                                   _ptr(u3), u3.stride(0) if u3 is not None else 0,
                                   u3.stride(1) if u3 is not None else 0, _ptr(q_index), n_sel,
                                   _ptr(o3), o3.stride(0), o3.stride(1), h_out, w_out, _ptr(err_flag),
                                   _stream(base.device)))
    return out


def var_attn_saliency(schedule, q, k, lse, step, softmax_scale=0.0, out=None):
    """Per-(batch, head) saliency [B, H, n_s] (fp32) of the positions of scale `step`.

    q [B, H, n_s, D] bf16 (the step's queries), k [B, H, >= off[step+1], D] bf16,
    lse [B, H, n_s] fp32 from var_attn_dense(..., step, step + 1, return_lse=True).
    """
    s = _as_schedule(schedule)
    _, n_s, kv_len = var_schedule_extent(s, step, step + 1)
    for name, t in (("q", q), ("k", k)):
        if t.dim() != 4 or not t.is_cuda or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a 4-D bf16 device tensor [batch, head, token, dim]")
    B, H, _, D = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D or k.device != q.device:
        raise ValueError("q and k disagree in batch, heads, head_dim or device")
    if q.shape[2] < n_s or k.shape[2] < kv_len:
        raise ValueError("q or k hold too few tokens for the step")
    if (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, n_s) or not lse.is_contiguous()
            or lse.device != q.device):
        raise ValueError(f"lse must be a contiguous fp32 tensor of shape {(B, H, n_s)} on q's device")
    if out is None:
        out = torch.empty((B, H, n_s), dtype=torch.float32, device=q.device)
    elif (out.dtype != torch.float32 or tuple(out.shape) != (B, H, n_s) or not out.is_contiguous()
          or out.device != q.device):
        raise ValueError(f"out must be a contiguous fp32 tensor of shape {(B, H, n_s)} on q's device")
    desc = AttnDesc(B, H, D, step, step + 1, float(softmax_scale), VAR_BF16, VAR_F32)
    _check(LIB.var_attn_saliency(ctypes.byref(s), ctypes.byref(desc), _ptr(q), _layout(q), _ptr(k), _layout(k),
                                 _ptr(lse), _ptr(out), _stream(q.device)))
    return out


def var_select_topk(saliency, h_src, w_src, h_dst, w_dst, n_keep, out=None):
    """Retained positions (int32 [n_keep], ascending) of the h_dst x w_dst grid.

    saliency: fp32 [..., h_src*w_src] contiguous; the leading dims are the maps
    (e.g. [B, H, n_s] from var_attn_saliency), summed in order.
    """
    n_src = h_src * w_src
    if saliency.dtype != torch.float32 or not saliency.is_contiguous() or not saliency.is_cuda:
        raise ValueError("saliency must be a contiguous fp32 device tensor")
    if saliency.shape[-1] != n_src:
        raise ValueError(f"saliency's last dim must be h_src*w_src = {n_src}")
    maps = saliency.numel() // n_src
    if out is None:
        out = torch.empty(max(0, int(n_keep)), dtype=torch.int32, device=saliency.device)
    elif out.dtype != torch.int32 or out.numel() < n_keep or not out.is_contiguous() or out.device != saliency.device:
        raise ValueError("out must be a contiguous int32 tensor with n_keep entries on saliency's device")
    _check(LIB.var_select_topk(maps, _ptr(saliency), h_src, w_src, h_dst, w_dst, int(n_keep),
                               _ptr(out) if n_keep > 0 else ctypes.c_void_p(0), _stream(saliency.device)))
    return out


def var_attn_block_mass(schedule, q, k, lse, step, softmax_scale=0.0, out=None):
    """Attention mass [B, H, n_qt, n_kt] (fp32) of the 64x64 tiles of step `step` (the decision scale).

    q [B, H, n_d, D] bf16 (the step's queries), k [B, H, >= off[step+1], D] bf16,
    lse [B, H, n_d] fp32 from var_attn_dense(..., step, step + 1, return_lse=True).
    """
    s = _as_schedule(schedule)
    _, n_d, L = var_schedule_extent(s, step, step + 1)
    B, H, _, D = q.shape
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or not q.is_cuda or k.device != q.device:
        raise ValueError("q and k must be bf16 tensors on one device")
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D or q.shape[2] < n_d or k.shape[2] < L:
        raise ValueError("q / k shapes do not fit the step")
    if (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, n_d) or not lse.is_contiguous()
            or lse.device != q.device):
        raise ValueError(f"lse must be a contiguous fp32 tensor of shape {(B, H, n_d)}")
    shape = (B, H, -(-n_d // 64), -(-L // 64))
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=q.device)
    elif tuple(out.shape) != shape or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous fp32 tensor of shape {shape}")
    desc = AttnDesc(B, H, D, step, step + 1, float(softmax_scale), VAR_BF16, VAR_F32)
    _check(LIB.var_attn_block_mass(ctypes.byref(s), ctypes.byref(desc), _ptr(q), _layout(q), _ptr(k), _layout(k),
                                   _ptr(lse), _ptr(out), _stream(q.device)))
    return out


def var_decision_tiles(mass, tau, out=None):
    """kept (uint8, same shape as mass [..., n_qt, n_kt]) of the decision scale."""
    if mass.dtype != torch.float32 or not mass.is_contiguous() or not mass.is_cuda or mass.dim() < 2:
        raise ValueError("mass must be a contiguous fp32 device tensor [..., n_qt, n_kt]")
    n_qt, n_kt = mass.shape[-2], mass.shape[-1]
    maps = mass.numel() // (n_qt * n_kt)
    if out is None:
        out = torch.empty(mass.shape, dtype=torch.uint8, device=mass.device)
    elif out.shape != mass.shape or out.dtype != torch.uint8 or not out.is_contiguous():
        raise ValueError("out must be a contiguous uint8 tensor shaped like mass")
    _check(LIB.var_decision_tiles(maps, n_qt, n_kt, _ptr(mass), float(tau), _ptr(out), _stream(mass.device)))
    return out


def var_mapped_tile_mask(schedule, decision_scale, step, kept_d, row_ptr=None, col_idx=None):
    """Per-map CSR of step `step`: row_ptr int32 [maps, n_qt+1], col_idx int32 [maps, n_qt*n_kt]."""
    s = _as_schedule(schedule)
    if kept_d.dtype != torch.uint8 or not kept_d.is_contiguous() or not kept_d.is_cuda or kept_d.dim() < 2:
        raise ValueError("kept_d must be a contiguous uint8 device tensor [..., n_qt_d, n_kt_d]")
    _, n_d, L_d = var_schedule_extent(s, decision_scale, decision_scale + 1)
    _, n_t, L_t = var_schedule_extent(s, step, step + 1)
    if kept_d.shape[-2:] != (-(-n_d // 64), -(-L_d // 64)):
        raise ValueError("kept_d's last two dims must be the decision step's tile counts")
    maps = kept_d.numel() // (kept_d.shape[-2] * kept_d.shape[-1])
    n_qt, n_kt = -(-n_t // 64), -(-L_t // 64)
    if row_ptr is None:
        row_ptr = torch.empty(maps, n_qt + 1, dtype=torch.int32, device=kept_d.device)
    if col_idx is None:
        col_idx = torch.empty(maps, n_qt * n_kt, dtype=torch.int32, device=kept_d.device)
    if (row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32 or tuple(row_ptr.shape) != (maps, n_qt + 1)
            or col_idx.dim() != 2 or col_idx.shape[0] != maps or not row_ptr.is_contiguous()
            or not col_idx.is_contiguous()):
        raise ValueError("row_ptr must be int32 [maps, n_qt+1] and col_idx int32 [maps, >= n_qt*n_kt], contiguous")
    _check(LIB.var_mapped_tile_mask(ctypes.byref(s), decision_scale, step, maps, _ptr(kept_d), _ptr(row_ptr),
                                    _ptr(col_idx), col_idx.shape[1], _stream(kept_d.device)))
    return row_ptr, col_idx


def var_attn_block_sparse_heads(schedule, q, k, v, q_scale_begin, q_scale_end, row_ptr, col_idx, out=None,
                                out_dtype=None, softmax_scale=0.0, q_index=None, return_lse=False, out_at_index=False):
    """Block-sparse attention with one CSR per (batch, head): row_ptr [B*H, n_qt+1], col_idx [B*H, stride]."""
    s, desc, out, lse, rows = _attn_common(schedule, q, k, v, q_scale_begin, q_scale_end, out, out_dtype,
                                           softmax_scale, q_index, return_lse, out_at_index=out_at_index)
    n_sel = rows if q_index is not None else 0
    if q_index is not None and n_sel == 0:
        return (out, lse) if return_lse else out
    B, H = q.shape[0], q.shape[1]
    n_qt = -(-rows // 64)
    if (row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32 or tuple(row_ptr.shape) != (B * H, n_qt + 1)
            or col_idx.dim() != 2 or col_idx.shape[0] != B * H or not row_ptr.is_contiguous()
            or not col_idx.is_contiguous() or row_ptr.device != q.device or col_idx.device != q.device):
        raise ValueError("row_ptr must be int32 [B*H, n_qt+1] and col_idx int32 [B*H, stride] on q's device")
    _check(LIB.var_attn_block_sparse_heads(ctypes.byref(s), ctypes.byref(desc), _ptr(q), _layout(q), _ptr(k),
                                           _layout(k), _ptr(v), _layout(v), _ptr(out), _layout(out), _ptr(lse),
                                           _ptr(q_index), n_sel, _ptr(row_ptr), _ptr(col_idx), col_idx.shape[1],
                                           _stream(q.device)))
    return (out, lse) if return_lse else out


def var_quantize_e4m3(x, codes=None, scale=None, first_token=0):
    """x bf16 [B, H, T, D] -> (codes uint8 [B, H, T, D], scale fp32 [B, H, ceil(T/64)]).

    value = e4m3(code) * scale of its 64-token tile.  With first_token > 0 only
    the tiles from first_token // 64 on are (re)written into the given
    codes / scale (the others keep their contents).
    """
    if x.dim() != 4 or not x.is_cuda or x.dtype != torch.bfloat16:
        raise ValueError("x must be a 4-D bf16 device tensor [batch, head, token, dim]")
    B, H, T, D = x.shape
    n_t = -(-T // 64)
    if codes is None:
        codes = torch.empty((B, H, T, D), dtype=torch.uint8, device=x.device)
    elif tuple(codes.shape) != (B, H, T, D) or codes.dtype != torch.uint8 or codes.device != x.device:
        raise ValueError(f"codes must be uint8 {(B, H, T, D)} on x's device")
    if scale is None:
        scale = torch.empty((B, H, n_t), dtype=torch.float32, device=x.device)
    elif (scale.dim() != 3 or tuple(scale.shape[:2]) != (B, H) or scale.shape[2] < n_t or scale.dtype != torch.float32
          or not scale.is_contiguous() or scale.device != x.device):
        raise ValueError(f"scale must be a contiguous fp32 tensor [B, H, >= {n_t}] on x's device")
    if T > first_token:
        _check(LIB.var_quantize_e4m3(B, H, T, D, _ptr(x), _layout(x), _ptr(codes), _layout(codes), _ptr(scale),
                                     scale.shape[2], int(first_token), _stream(x.device)))
    return codes, scale


def _scale_arg(t, B, H, dev, name):
    if (t.dim() != 3 or tuple(t.shape[:2]) != (B, H) or t.dtype != torch.float32 or not t.is_contiguous()
            or t.device != dev):
        raise ValueError(f"{name} must be a contiguous fp32 tensor [B, H, tiles] on q's device")
    return _ptr(t), t.shape[2]


def var_attn_dense_e4m3(schedule, q, k, k_scale, v, q_scale_begin, q_scale_end, out=None, out_dtype=None,
                        softmax_scale=0.0, q_index=None, return_lse=False, n_splits=1, workspace=None, out_at_index=False):
    """var_attn_dense with e4m3 logits: k as e4m3 codes (uint8) with tile scales [B, H, tiles]
    (var_quantize_e4m3); q bf16, quantised in the call per 64 output rows."""
    s, desc, out, lse, rows = _attn_common(schedule, q, k, v, q_scale_begin, q_scale_end, out, out_dtype,
                                           softmax_scale, q_index, return_lse, qk_codes=True, out_at_index=out_at_index)
    n_sel = rows if q_index is not None else 0
    if q_index is not None and n_sel == 0:
        return (out, lse) if return_lse else out
    B, H = q.shape[0], q.shape[1]
    wp, wb = _ws_args(n_splits, workspace)
    _check(LIB.var_attn_dense_e4m3(ctypes.byref(s), ctypes.byref(desc), _ptr(q), _layout(q), _ptr(k), _layout(k),
                                   *_scale_arg(k_scale, B, H, q.device, "k_scale"), _ptr(v), _layout(v), _ptr(out),
                                   _layout(out), _ptr(lse), _ptr(q_index), n_sel, int(n_splits), wp, wb,
                                   _stream(q.device)))
    return (out, lse) if return_lse else out


def var_attn_block_sparse_e4m3(schedule, q, k, k_scale, v, q_scale_begin, q_scale_end, row_ptr, col_idx,
                               out=None, out_dtype=None, softmax_scale=0.0, q_index=None, return_lse=False, out_at_index=False):
    """Block-sparse attention with e4m3 logits (as var_attn_dense_e4m3).  row_ptr / col_idx 1-D: one CSR
    for every (batch, head); 2-D [B*H, n_qt+1] / [B*H, stride]: one CSR per (batch, head)."""
    s, desc, out, lse, rows = _attn_common(schedule, q, k, v, q_scale_begin, q_scale_end, out, out_dtype,
                                           softmax_scale, q_index, return_lse, qk_codes=True, out_at_index=out_at_index)
    n_sel = rows if q_index is not None else 0
    if q_index is not None and n_sel == 0:
        return (out, lse) if return_lse else out
    B, H = q.shape[0], q.shape[1]
    n_qt = -(-rows // 64)
    for name, t in (("row_ptr", row_ptr), ("col_idx", col_idx)):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous int32 tensor on q's device")
    if row_ptr.dim() == 1:
        if row_ptr.numel() < n_qt + 1 or col_idx.dim() != 1:
            raise ValueError(f"a shared CSR needs row_ptr of {n_qt + 1} entries and a 1-D col_idx")
        stride = 0
    else:
        if tuple(row_ptr.shape) != (B * H, n_qt + 1) or col_idx.dim() != 2 or col_idx.shape[0] != B * H:
            raise ValueError("per-head CSR: row_ptr int32 [B*H, n_qt+1], col_idx int32 [B*H, stride]")
        stride = col_idx.shape[1]
    _check(LIB.var_attn_block_sparse_e4m3(ctypes.byref(s), ctypes.byref(desc), _ptr(q), _layout(q), _ptr(k),
                                          _layout(k), *_scale_arg(k_scale, B, H, q.device, "k_scale"), _ptr(v),
                                          _layout(v), _ptr(out), _layout(out), _ptr(lse), _ptr(q_index), n_sel,
                                          _ptr(row_ptr), _ptr(col_idx), stride, _stream(q.device)))
    return (out, lse) if return_lse else out
