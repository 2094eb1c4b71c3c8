"""Plain float64 attention: the definition the tiled kernel must reach.

TEST INFRASTRUCTURE ONLY (see the package docstring); the product path never
uses this module.

For every batch b, head h and query row i (the problem statement of [P1]
"왜 필요한가" and the scaled form of [P3] "N×N 행렬은 꼭 저장해야 할까" and of
the [P2] tiling pseudocode):

    s_j = scale * <q_i, k_j>            for every allowed key j
    m   = max_j s_j                      (safe softmax, [P1] "Online Softmax 개념")
    e_j = exp(s_j - m)
    l   = sum_j e_j
    P_ij = e_j / l                       (softmax definition, [P1] "왜 필요한가")
    O_i = sum_j P_ij v_j
    L_i = m + log(l)                     (logsumexp, [P1] FA2 section, epilogue eq.)

A key j is allowed when j < N, and additionally j <= i under the causal mask
(the lower-triangular mask that lets FA2 skip key blocks above the diagonal,
[P2] "v2와 v3"). ``L`` is the natural log of the scaled, masked scores, so that
exp(S_ij - L_i) = P_ij holds exactly as the LSE identity in the [P1] FA2
section states.

Rows are independent ([P1] FA2 section: row blocks do not depend on each
other), so computing the rows in chunks on several threads is still the plain
definition; no blocking over keys is done.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = ["attention", "attention_rows", "default_workers"]


def default_workers() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _head_rows(qh, kh, vh, scale, causal, idx):
    """O and L for the query rows ``idx`` of one head (all float64)."""
    n_keys = kh.shape[0]
    if causal:
        # keys after the last requested row can never be allowed
        n_keys = min(n_keys, int(idx.max()) + 1)
    k_used = kh[:n_keys]
    s = scale * (qh[idx] @ k_used.T)
    if causal:
        allowed = np.arange(n_keys)[None, :] <= idx[:, None]
        s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    p = e / l[:, None]
    o = p @ vh[:n_keys]
    return o, m + np.log(l)


def attention_rows(q, k, v, scale, causal, heads, rows, workers=None, chunk=256):
    """O and L for selected heads and query rows.

    q, k: float64-compatible arrays [B, H, N, d]; v: [B, H, N, dv].
    heads:   sequence of (b, h) pairs.
    rows:    1-D integer array of query indices, used for every listed head.
    Returns (O [len(heads), len(rows), dv], L [len(heads), len(rows)]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    d = v.shape[-1]
    out_o = np.empty((len(heads), len(rows), d), dtype=np.float64)
    out_l = np.empty((len(heads), len(rows)), dtype=np.float64)
    if len(rows) == 0 or len(heads) == 0:
        return out_o, out_l
    tasks = []
    for hi, (b, h) in enumerate(heads):
        for c0 in range(0, len(rows), chunk):
            tasks.append((hi, b, h, c0, min(c0 + chunk, len(rows))))

    def run(t):
        hi, b, h, c0, c1 = t
        o, lse = _head_rows(q[b, h], k[b, h], v[b, h], scale, causal, rows[c0:c1])
        out_o[hi, c0:c1] = o
        out_l[hi, c0:c1] = lse

    nw = workers or default_workers()
    if nw == 1 or len(tasks) == 1:
        for t in tasks:
            run(t)
    else:
        try:
            from threadpoolctl import threadpool_limits
        except ImportError:  # pragma: no cover
            threadpool_limits = None
        if threadpool_limits is not None:
            with threadpool_limits(limits=1):
                with ThreadPoolExecutor(max_workers=nw) as ex:
                    list(ex.map(run, tasks))
        else:  # pragma: no cover
            with ThreadPoolExecutor(max_workers=nw) as ex:
                list(ex.map(run, tasks))
    return out_o, out_l


def attention(q, k, v, scale, causal, workers=None):
    """O [B, H, N, d] and L [B, H, N] for every row, in float64."""
    q = np.asarray(q, dtype=np.float64)
    B, H, N, _ = q.shape
    d = np.shape(v)[-1]
    heads = [(b, h) for b in range(B) for h in range(H)]
    o, lse = attention_rows(q, k, v, scale, causal, heads, np.arange(N), workers)
    return o.reshape(B, H, N, d), lse.reshape(B, H, N)
