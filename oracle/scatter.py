"""Structural reconstruction of a pruned grid (oracle; test infrastructure only).

"ARVAR: Accelerating Visual Autoregressive Model via Attention Retrospect",
Key Design 3, Equations (8)-(9): the full output of the current step is an
earlier step's output interpolated to the current grid, with the freshly
computed rows written over the retained positions I_T.  Scatter overwrites; it
never adds old and new values.

The page leaves the interpolation mode open.  Reading taken: plain nearest
neighbour with source index floor(dst * in / out) on each axis (the classic
"nearest" rule; for 48 -> 64 it picks the same sources as any other common
floor-based nearest).  Values are copied bit for bit, so the function works on
any dtype.
"""

import numpy as np


def nearest_source_index(h_in, w_in, h_out, w_out):
    """Row-major source token of every destination token of an h_out x w_out grid."""
    ys = (np.arange(h_out, dtype=np.int64) * h_in) // h_out
    xs = (np.arange(w_out, dtype=np.int64) * w_in) // w_out
    return (ys[:, None] * w_in + xs[None, :]).reshape(-1)


def scatter_restore(base, h_in, w_in, upd, q_index, h_out, w_out):
    """out[..., t, :] = base[..., up(t), :]; then out[..., q_index[i], :] = upd[..., i, :].

    base [..., h_in*w_in, E], upd [..., n_sel, E], q_index ints [n_sel] (unique,
    in [0, h_out*w_out)).  Returns out [..., h_out*w_out, E] with base's dtype.
    """
    base = np.asarray(base)
    upd = np.asarray(upd)
    q_index = np.asarray(q_index, dtype=np.int64)
    if base.shape[-2] != h_in * w_in:
        raise ValueError("base does not hold h_in*w_in rows")
    if upd.shape[-2] != q_index.size:
        raise ValueError("upd rows != n_sel")
    n_out = h_out * w_out
    if q_index.size and (q_index.min() < 0 or q_index.max() >= n_out):
        raise ValueError("q_index out of range")
    if np.unique(q_index).size != q_index.size:
        raise ValueError("q_index has duplicates")
    src = nearest_source_index(h_in, w_in, h_out, w_out)
    out = base[..., src, :].copy()
    out[..., q_index, :] = upd.astype(base.dtype, copy=False)
    return out
