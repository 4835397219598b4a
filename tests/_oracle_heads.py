"""The oracle's attention for every (batch, head) of a full-size call, one pair per thread.

Test-side parallelism only: each thread calls oracle.attention on a one-pair
slice, unchanged.  NumPy's element-wise passes (the mask, exp, sums) run
single-threaded inside one call, so running pairs side by side, with BLAS
held to a few threads each, finishes a 32-pair 1024px step in seconds.
"""

import concurrent.futures
import os

import numpy as np

import oracle


def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def attention_all_heads(q, k, v, h, w, q_scale_begin, q_scale_end, return_lse=False, **kw):
    """oracle.attention over [B, H, ...] inputs, computed pair by pair in parallel."""
    B, H = q.shape[:2]
    pairs = [(b, hh) for b in range(B) for hh in range(H)]
    workers = _workers()

    def one(bh):
        b, hh = bh
        return oracle.attention(q[b:b + 1, hh:hh + 1], k[b:b + 1, hh:hh + 1], v[b:b + 1, hh:hh + 1], h, w,
                                q_scale_begin, q_scale_end, return_lse=True, **kw)

    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"):
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            res = list(ex.map(one, pairs))
    n = res[0][0].shape[2]
    D = res[0][0].shape[3]
    out = np.empty((B, H, n, D))
    lse = np.empty((B, H, n))
    for (b, hh), (o, l) in zip(pairs, res):
        out[b, hh] = o[0, 0]
        lse[b, hh] = l[0, 0]
    return (out, lse) if return_lse else out
