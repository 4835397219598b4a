"""Attention-guided choice of the positions to recompute (oracle; test infrastructure only).

"ARVAR: Accelerating Visual Autoregressive Model via Attention Retrospect",
Key Design 2 (attention-guided pruning) and A Worked Example: at the large
step T the model does not form a new attention matrix.  It takes the
attention of the same layer at the earlier, smaller step T-M, keeps its
self-attention part, reduces it to one saliency score per position of that
step's grid, interpolates the map to the grid of step T, and Top-K of the
interpolated map gives the retained indices I_T (gathered for the pruned
attention, scattered back by the reconstruction of Key Design 3).

The page itself says the axis of the reduction, the normalisation of the
extracted block, the aggregation over heads and the interpolation mode are
not specified.  Readings taken:

* Self-attention part: the columns of the step's attention weights P (each
  row normalised over every key the query sees, i.e. the weights the layer
  actually used) that belong to the step's own tokens: a square n_s x n_s
  block.
* Reduction: the mean over the step's queries of each column of that block
  (the attention a position receives).  A mean along rows of a row-normalised
  square matrix would be the same for every row, which the page rules out.
* Heads and the two CFG branches: one saliency map per (batch, head).  The
  selection adds the maps in order m = 0, 1, ... in float32 arithmetic, so
  that its integer decisions are taken in the precision of the device code
  (the ranking by a sum equals the ranking by the mean).
* Interpolation: nearest, source floor(dst * in / out) per axis, the same
  rule as the reconstruction.
* Top-K order: larger score first, equal scores by lower position; the
  retained positions are returned in ascending order.

Saliency is computed in float64 from the definition (logits, row softmax over
all visible keys, column mean of the own-scale block).
"""

import math

import numpy as np

from .schedule import offsets
from .scatter import nearest_source_index


def saliency(q, k, h, w, step, softmax_scale=None):
    """Per-(batch, head) saliency of the positions of scale `step`.

    q  [B, H, n_s, D]   the queries of scale `step` (tokens off[step] ...).
    k  [B, H, >= L, D]  the key cache, L = off[step + 1]; a query of scale
                        `step` sees every key u < L.
    Returns S [B, H, n_s] float64 with
        S[b, h, u] = (1 / n_s) * sum_i P[b, h, i, off[step] + u],
        P[b, h, i, :] = softmax(scale * q_i K^T) over the L visible keys.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    B, H, n_given, D = q.shape
    off = offsets(h, w)
    s = int(step)
    if not (0 <= s < len(h)):
        raise ValueError("bad step")
    L = off[s + 1]
    n_s = off[s + 1] - off[s]
    if n_given < n_s or k.shape[2] < L:
        raise ValueError("q or k too short for the step")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    out = np.zeros((B, H, n_s), dtype=np.float64)
    for bi in range(B):
        for hi in range(H):
            Q = q[bi, hi, :n_s, :].astype(np.float64)
            K = k[bi, hi, :L, :].astype(np.float64)
            logits = scale * (Q @ K.T)                    # [n_s, L], every key visible
            p = np.exp(logits - logits.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            out[bi, hi] = p[:, off[s]:L].mean(axis=0)     # own-scale block, column mean
    return out


def selection_scores(maps, h_src, w_src, h_dst, w_dst):
    """Score of every destination position: float32 sum of the maps in order, nearest-upsampled.

    maps [n_maps, h_src*w_src] float32 saliency maps (as the device produced them).
    Returns float32 [h_dst*w_dst].
    """
    maps = np.asarray(maps, dtype=np.float32).reshape(-1, h_src * w_src)
    acc = np.zeros(h_src * w_src, dtype=np.float32)
    for m in range(maps.shape[0]):
        acc = np.add(acc, maps[m], dtype=np.float32)      # one IEEE single add per element, in map order
    return acc[nearest_source_index(h_src, w_src, h_dst, w_dst)]


def select_positions(maps, h_src, w_src, h_dst, w_dst, n_keep):
    """Retained positions I_T: the n_keep best destination positions, ascending (int32).

    Best = larger score first, equal scores by lower position.  Scores must not
    be NaN; -0.0 counts as 0.
    """
    score = selection_scores(maps, h_src, w_src, h_dst, w_dst).astype(np.float64)
    n_dst = score.size
    if not (0 <= n_keep <= n_dst):
        raise ValueError("n_keep outside [0, h_dst*w_dst]")
    order = np.lexsort((np.arange(n_dst), -score))         # primary: score descending; then position
    return np.sort(order[:n_keep]).astype(np.int32)
