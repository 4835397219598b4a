"""Exact block-causal next-scale attention in float64 (oracle; test infrastructure only).

What is computed, and where it comes from:

* Visibility.  "SparVAR: Exploring Sparsity in Visual AutoRegressive Modeling
  for Training-Free Acceleration" (abstract) says that at every step the model
  attends to all tokens across the historical scales; "ARVAR: Accelerating
  Visual Autoregressive Model via Attention Retrospect" (Background &
  Motivation) says each step predicts a whole grid at once with a KV cache.
  Reading taken: a query of scale q sees every key u with sigma(u) <= q —
  all earlier scales and its whole own scale (no causal order inside a scale).
* The score is plain softmax attention (method tags "Attention" and "Softmax"
  on the LiteVAR record; the FlashAttention baselines of the ARVAR page
  compute exact attention): O = softmax(s * Q K^T) V with s = 1/sqrt(D) unless
  given.  No bias, no dropout.
* Block-sparse variant ("SparVAR ...", abstract: block-wise sparse
  attention).  Given a tile mask kept[r, c], a query that is the i-th row of
  the call (tile r = i // tile_q) additionally sees only keys u whose key tile
  c = u // tile_k is kept.  Inside a kept tile every visible pair is attended
  (the sparsity is tile-granular).
* Pruned queries ("ARVAR ...", Key Design 2: the retained indices gather the
  important tokens).  With q_index the call's rows are the query rows
  q_index[0], q_index[1], ... of the step; each keeps its own position, hence
  its own scale and visibility.

The arithmetic is the definition written out: logits with a float64 matrix
product, the row max, exp, the row sum and a float64 product with V.  A row
that sees no key returns O = 0 and LSE = -inf.
"""

import math

import numpy as np

from .schedule import offsets, scale_of_tokens


def attention(q, k, v, h, w, q_scale_begin, q_scale_end, softmax_scale=None,
              q_index=None, kept=None, tile_q=64, tile_k=64, rows=None,
              return_lse=False, return_probs=False):
    """Attention of the queries of scales [q_scale_begin, q_scale_end).

    q       [B, H, n_q, D]  query block of the call; row j is token off[b] + j,
                            n_q = off[e] - off[b].
    k, v    [B, H, >= L, D] key / value cache; only tokens [0, L), L = off[e],
                            are read.
    q_index optional ints [n_sel]: the call's rows are q[:, :, q_index[i]].
    kept    optional bool [n_qt, n_kt]: tile mask; row i of the call lies in
            query tile i // tile_q, key u in key tile u // tile_k.
    rows    optional subset (indices into the call's rows) to evaluate; the
            tile of a row is still taken from its index among all call rows.

    Returns O [B, H, n_eval, D] (float64); with return_lse also LSE
    [B, H, n_eval] (natural log); with return_probs also the row-normalised
    weights P [B, H, n_eval, L].
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H, n_q_given, D = q.shape
    off = offsets(h, w)
    b, e = int(q_scale_begin), int(q_scale_end)
    if not (0 <= b < e <= len(h)):
        raise ValueError("bad scale range")
    L = off[e]
    n_q = off[e] - off[b]
    if n_q_given < n_q:
        raise ValueError("q holds fewer rows than the scales' tokens")
    if k.shape[2] < L or v.shape[2] < L:
        raise ValueError("k/v hold fewer than L tokens")
    sigma = scale_of_tokens(h, w)[:L]

    call_pos = np.arange(n_q) if q_index is None else np.asarray(q_index, dtype=np.int64)
    if call_pos.size and (call_pos.min() < 0 or call_pos.max() >= n_q):
        raise ValueError("q_index out of range")
    eval_rows = np.arange(call_pos.size) if rows is None else np.asarray(rows, dtype=np.int64)
    pos = call_pos[eval_rows]
    tok = off[b] + pos

    # visibility: sigma(key) <= sigma(query)
    vis = sigma[None, :] <= sigma[tok][:, None]
    if kept is not None:
        kept = np.asarray(kept, dtype=bool)
        key_tile = np.arange(L) // tile_k
        vis &= kept[eval_rows // tile_q][:, key_tile]

    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    n_eval = eval_rows.size
    out = np.zeros((B, H, n_eval, D), dtype=np.float64)
    lse = np.full((B, H, n_eval), -np.inf, dtype=np.float64)
    probs = np.zeros((B, H, n_eval, L), dtype=np.float64) if return_probs else None

    for bi in range(B):
        for hi in range(H):
            Q = q[bi, hi, pos, :].astype(np.float64)
            K = k[bi, hi, :L, :].astype(np.float64)
            V = v[bi, hi, :L, :].astype(np.float64)
            s = scale * (Q @ K.T)
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, initial=-np.inf)
            has = np.isfinite(m)
            m_safe = np.where(has, m, 0.0)
            p = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 for hidden keys
            l = p.sum(axis=1)
            o = p @ V
            denom = np.where(has, l, 1.0)
            out[bi, hi] = np.where(has[:, None], o / denom[:, None], 0.0)
            lse[bi, hi] = np.where(has, m_safe + np.log(denom), -np.inf)
            if return_probs:
                probs[bi, hi] = np.where(has[:, None], p / denom[:, None], 0.0)

    res = [out]
    if return_lse:
        res.append(lse)
    if return_probs:
        res.append(probs)
    return res[0] if len(res) == 1 else tuple(res)
