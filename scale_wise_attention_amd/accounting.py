"""Algorithmic work and traffic of next-scale attention launches (benchmark bookkeeping).

Counting rules:
* FLOPs = 4 * D * B * H * (attended pairs): one multiply-add per element of
  q.k and one per element of p.v.  Exponentials, maxima and sums are not
  counted.  Dense: every visible (query, key) pair.  Block-sparse: every
  visible pair inside a kept tile (only computed tiles count).
* Bytes = Q rows read + K and V prefix read once + O written once, per
  (batch, head), at the tensors' element sizes.
"""


def step_sizes(grids_h, grids_w, step):
    n = [a * b for a, b in zip(grids_h, grids_w)]
    first = sum(n[:step])
    return n[step], first + n[step]      # (queries of the step, keys visible to them)


def dense_step_flops(wl, step, rows=None):
    n_q, L = step_sizes(wl.h, wl.w, step)
    n = n_q if rows is None else rows
    return 4.0 * wl.head_dim * wl.batch * wl.heads * n * L


def dense_step_bytes(wl, step, in_bytes=2, out_bytes=2, rows=None):
    n_q, L = step_sizes(wl.h, wl.w, step)
    n = n_q if rows is None else rows
    per_bh = n * wl.head_dim * in_bytes + 2 * L * wl.head_dim * in_bytes + n * wl.head_dim * out_bytes
    return float(per_bh * wl.batch * wl.heads)


def sparse_pairs(row_ptr, col_idx, n_rows, kv_len, tile_q=64, tile_k=64):
    """Visible pairs inside kept tiles for a single-scale (step) call: every key < kv_len is visible."""
    pairs = 0
    for r in range(len(row_ptr) - 1):
        rows_in_tile = min(tile_q, n_rows - r * tile_q)
        for c in col_idx[row_ptr[r]:row_ptr[r + 1]]:
            keys = min(tile_k, kv_len - int(c) * tile_k)
            pairs += rows_in_tile * keys
    return pairs


def sparse_step_flops(wl, row_ptr, col_idx, n_rows, kv_len):
    return 4.0 * wl.head_dim * wl.batch * wl.heads * sparse_pairs(row_ptr, col_idx, n_rows, kv_len)


def scatter_bytes(maps, row_bytes, n_sel, n_out):
    """Each output row written once and read once from its single source."""
    return float(maps * n_out * row_bytes * 2)
