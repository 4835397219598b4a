"""Per-head sparse pattern predicted from a decision scale (oracle; test infrastructure only).

"SparVAR: Exploring Sparsity in Visual AutoRegressive Modeling for
Training-Free Acceleration", abstract: the sparse attention pattern of the
later, high-resolution scales is predicted dynamically from a sparse decision
scale, and the pattern of a large scale is built self-similar to it through an
index mapping between scales.  The abstract gives no formulas; the readings
taken here are:

* Attention mass at the decision scale d (a step computed in full, whose LSE
  is known): for each (batch, head), query tile r (64 consecutive rows of the
  step) and key tile c (64 consecutive cache tokens of [0, L_d)),
  mass[r, c] = sum over i in r, u in c of P[i, u], with P the step's attention
  weights (each row sums to 1).
* Decision: per (batch, head, r), the key tiles in order of decreasing mass
  (equal masses by lower c) are kept while the mass already kept is below
  tau times the row tile's total.  The sums are float32, in that order, the
  total in ascending c, so that the integer decision is taken in the
  precision of the device code.
* Index mapping to a later step T >= d: query (y, x) of scale T stands for
  position (floor(y*h_d/h_T), floor(x*w_d/w_T)) of scale d, i.e. for the
  decision row tile of that token.  A key of scale j <= d stands for itself
  (the decision step saw the same cached token); a key (y, x) of scale j > d
  stands for (floor(y*h_d/h_j), floor(x*w_d/w_j)) of scale d.  Tile (R, C) of
  step T is kept when some query of R and key of C stand for a kept decision
  pair.  Every key of [0, L_T) is visible to the queries of step T.
"""

import math

import numpy as np

from .schedule import offsets, token_coords


def block_mass(q, k, h, w, d, tile=64, softmax_scale=None):
    """mass [B, H, n_qt, n_kt] (float64) of the attention of step d (queries of scale d, keys [0, L_d))."""
    q = np.asarray(q)
    k = np.asarray(k)
    B, H, n_given, D = q.shape
    off = offsets(h, w)
    L = off[d + 1]
    n = off[d + 1] - off[d]
    if n_given < n or k.shape[2] < L:
        raise ValueError("q or k too short for the step")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    n_qt, n_kt = -(-n // tile), -(-L // tile)
    out = np.zeros((B, H, n_qt, n_kt))
    for b in range(B):
        for hh in range(H):
            logits = scale * (q[b, hh, :n].astype(np.float64) @ k[b, hh, :L].astype(np.float64).T)
            p = np.exp(logits - logits.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            for r in range(n_qt):
                rows = p[r * tile:(r + 1) * tile]
                for c in range(n_kt):
                    out[b, hh, r, c] = rows[:, c * tile:(c + 1) * tile].sum()
    return out


def decision_tiles(mass, tau):
    """kept [..., n_qt, n_kt] (bool) from float32 masses [..., n_qt, n_kt]."""
    mass = np.asarray(mass, dtype=np.float32)
    tau = np.float32(tau)
    kept = np.zeros(mass.shape, dtype=bool)
    flat = mass.reshape(-1, mass.shape[-1])
    kflat = kept.reshape(-1, mass.shape[-1])
    n = mass.shape[-1]
    for row in range(flat.shape[0]):
        m = flat[row]
        total = np.float32(0.0)
        for c in range(n):
            total = np.float32(total + m[c])
        target = np.float32(tau * total)
        order = sorted(range(n), key=lambda c: (-float(m[c]), c))
        cum = np.float32(0.0)
        for c in order:
            if cum < target:
                kflat[row, c] = True
            cum = np.float32(cum + m[c])
    return kept


def mapped_tile_mask(h, w, d, T, kept_d, tile=64):
    """kept_T [maps, n_qt_T, n_kt_T] (bool) for step T from the decision tiles of step d (pair enumeration)."""
    kept_d = np.asarray(kept_d, dtype=bool)
    maps = kept_d.shape[0]
    off = offsets(h, w)
    if not (0 <= d <= T < len(h)):
        raise ValueError("need 0 <= d <= T < num_scales")
    sigma, y, x = token_coords(h, w)
    L = off[T + 1]
    n_t = off[T + 1] - off[T]
    n_qt, n_kt = -(-n_t // tile), -(-L // tile)
    # decision row of each query of step T
    qy, qx = y[off[T]:L], x[off[T]:L]
    q_dec = (qy * h[d] // h[T]) * w[d] + (qx * w[d] // w[T])            # index inside scale d
    q_tile = q_dec // tile
    # decision token of each key of [0, L_T)
    u = np.arange(L)
    js = sigma[:L]
    hj = np.asarray(h)[js]
    wj = np.asarray(w)[js]
    mapped = off[d] + (y[:L] * h[d] // hj) * w[d] + (x[:L] * w[d] // wj)
    k_dec = np.where(js <= d, u, mapped)
    k_tile = k_dec // tile
    key_tile_T = u // tile
    out = np.zeros((maps, n_qt, n_kt), dtype=bool)
    for m in range(maps):
        for i in range(n_t):
            sel = kept_d[m, q_tile[i]][k_tile]          # keys whose decision pair is kept
            out[m, i // tile, np.unique(key_tile_T[sel])] = True
    return out
