"""Scale schedule bookkeeping (oracle; test infrastructure only).

Next-scale prediction emits one whole h_k x w_k token grid per step
("ARVAR: Accelerating Visual Autoregressive Model via Attention Retrospect",
Background & Motivation; "SparVAR ...", abstract).  The tokens of one grid are
numbered row-major and the grids are concatenated in scale order, so token t
belongs to scale sigma(t) and sits at (y(t), x(t)) inside that grid.
"""

import numpy as np


def offsets(h, w):
    """off[k] = number of tokens in scales 0..k-1; off[K] = total tokens."""
    if len(h) != len(w):
        raise ValueError("h and w must have the same length")
    off = [0]
    for hk, wk in zip(h, w):
        off.append(off[-1] + int(hk) * int(wk))
    return off


def scale_of_tokens(h, w):
    """sigma[t] for every token t of the concatenated sequence (int64 array)."""
    parts = [np.full(int(hk) * int(wk), k, dtype=np.int64)
             for k, (hk, wk) in enumerate(zip(h, w))]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def token_coords(h, w):
    """(sigma, y, x) arrays over the concatenated sequence, row-major per scale."""
    sig, ys, xs = [], [], []
    for k, (hk, wk) in enumerate(zip(h, w)):
        hk, wk = int(hk), int(wk)
        yy, xx = np.meshgrid(np.arange(hk), np.arange(wk), indexing="ij")
        sig.append(np.full(hk * wk, k, dtype=np.int64))
        ys.append(yy.reshape(-1).astype(np.int64))
        xs.append(xx.reshape(-1).astype(np.int64))
    if not sig:
        z = np.zeros(0, dtype=np.int64)
        return z, z, z
    return np.concatenate(sig), np.concatenate(ys), np.concatenate(xs)
