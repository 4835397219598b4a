"""Tile mask for block-sparse next-scale attention (oracle; test infrastructure only).

"SparVAR: Exploring Sparsity in Visual AutoRegressive Modeling for
Training-Free Acceleration" (abstract) names the properties the sparse pattern
uses — strong attention sinks, pronounced locality, an index mapping between
scales — and a block-wise sparse kernel.  The concrete rule taken here (the
1024px sparse workload's rule) is:

  a (query, key) pair is *selected* when the key is visible to the query
  (sigma(key) <= sigma(query)) and either
    * the key lies in one of the first ``sink_scales`` scales (sink), or
    * the key lies in a scale j >= ``local_from_scale`` and its grid position
      is within the window of the query's position mapped into scale j:
          |y_q * h_j / h_q - y_k| <= radius_y  and  |x_q * w_j / w_q - x_k| <= radius_x,
      evaluated exactly in integers by multiplying through by h_q (w_q):
          |y_q * h_j - y_k * h_q| <= radius_y * h_q,  same for x with w.

  Tile (r, c) is kept when at least one selected pair has its query among the
  call's rows of query tile r (rows r*tile_q .. r*tile_q + tile_q - 1) and its
  key in key tile c (tokens c*tile_k .. c*tile_k + tile_k - 1, clipped to L).

This module computes the mask by enumerating every (query row, key) pair — the
brute-force form of the rule — and then lists the kept key tiles of each row in
ascending order (CSR).
"""

import numpy as np

from .schedule import offsets, token_coords


def tile_mask(h, w, q_scale_begin, q_scale_end, tile_q=64, tile_k=64,
              sink_scales=7, local_from_scale=7, radius_y=2, radius_x=2,
              q_index=None):
    """Boolean kept[n_qt, n_kt] for the call's query rows against keys [0, L)."""
    off = offsets(h, w)
    b, e = int(q_scale_begin), int(q_scale_end)
    if not (0 <= b < e <= len(h)):
        raise ValueError("bad scale range")
    L = off[e]
    n_q = off[e] - off[b]
    sigma, y, x = token_coords(h, w)
    sigma, y, x = sigma[:L], y[:L], x[:L]
    hs = np.asarray(h, dtype=np.int64)
    ws = np.asarray(w, dtype=np.int64)
    hj, wj = hs[sigma], ws[sigma]          # grid size of each key's scale

    call_pos = np.arange(n_q) if q_index is None else np.asarray(q_index, dtype=np.int64)
    n_rows = call_pos.size
    n_qt = -(-n_rows // tile_q)
    n_kt = -(-L // tile_k)
    kept = np.zeros((n_qt, n_kt), dtype=bool)
    key_tile = np.arange(L) // tile_k
    is_sink = sigma < sink_scales
    is_local_scale = sigma >= local_from_scale

    for i in range(n_rows):
        t = off[b] + int(call_pos[i])
        qs = int(sigma[t])
        hq, wq = int(hs[qs]), int(ws[qs])
        yq, xq = int(y[t]), int(x[t])
        visible = sigma <= qs
        in_window = (np.abs(yq * hj - y * hq) <= radius_y * hq) & \
                    (np.abs(xq * wj - x * wq) <= radius_x * wq)
        selected = visible & (is_sink | (is_local_scale & in_window))
        kept[i // tile_q, np.unique(key_tile[selected])] = True
    return kept


def mask_to_csr(kept):
    """CSR of a boolean tile mask: row_ptr int32 [n_qt + 1], col_idx int32, ascending per row."""
    kept = np.asarray(kept, dtype=bool)
    counts = kept.sum(axis=1)
    row_ptr = np.zeros(kept.shape[0] + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.nonzero(kept)[1].astype(np.int32)   # row-major order => ascending c per row
    return row_ptr, col_idx


def csr_to_mask(row_ptr, col_idx, n_kt):
    """Inverse of mask_to_csr."""
    row_ptr = np.asarray(row_ptr)
    col_idx = np.asarray(col_idx)
    n_qt = row_ptr.size - 1
    kept = np.zeros((n_qt, n_kt), dtype=bool)
    for r in range(n_qt):
        kept[r, col_idx[row_ptr[r]:row_ptr[r + 1]]] = True
    return kept
