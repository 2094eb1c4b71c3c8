"""The pages' online-softmax algorithm, step by step, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring). These functions follow
the algorithm in the order and notation the pages give it, so that the pages'
own claims can be checked: that the running sum ends equal to the safe-softmax
denominator, that block statistics merge with an exp(m_old - m_new) rescale,
and that the FA1 and FA2 loop orders reach the plain definition for every
block split.

Notation ([P1]): m is the running row maximum, l ("ℓ") the running sum of
exponentials relative to m, O~ the unnormalised output accumulator, alpha the
rescale of the old state, beta the rescale of the current block (FA1 only).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "online_softmax_scalar", "block_stats", "merge_stats", "split_rows",
    "fa2_forward", "fa1_forward",
]


def online_softmax_scalar(x):
    """The scalar recurrence of [P1] "Online Softmax 개념" (also [P2]
    "Online Softmax: 결합법칙이 ..."): after element x_j,
    m_j = max(m_{j-1}, x_j) and l_j = l_{j-1} * exp(m_{j-1} - m_j) + exp(x_j - m_j),
    starting from m_0 = -inf, l_0 = 0. Returns the list of (m_j, l_j)."""
    m, l = -math.inf, 0.0
    states = []
    for xj in x:
        m_new = max(m, float(xj))
        carry = 0.0 if m == -math.inf else l * math.exp(m - m_new)
        l = carry + math.exp(float(xj) - m_new)
        m = m_new
        states.append((m, l))
    return states


def block_stats(x):
    """(m, l) of one block: its maximum and its exponential sum relative to it."""
    x = np.asarray(x, dtype=np.float64)
    m = float(x.max())
    return m, float(np.exp(x - m).sum())


def merge_stats(a, b):
    """Merge two blocks' (m, l) on a common reference: the larger maximum wins and
    each sum is rescaled by exp(own max - new max) ([P1] "Online Softmax 개념",
    block form; [P3] "소프트맥스는 나누어 계산할 수 있다", the exp(2-4) step)."""
    (ma, la), (mb, lb) = a, b
    m = max(ma, mb)
    return m, la * math.exp(ma - m) + lb * math.exp(mb - m)


def split_rows(n, sizes):
    """Turn block sizes (a composition of n) into [start, stop) ranges."""
    if sum(sizes) != n or any(s <= 0 for s in sizes):
        raise ValueError(f"block sizes {sizes} are not a composition of {n}")
    out, s = [], 0
    for size in sizes:
        out.append((s, s + size))
        s += size
    return out


def _scores(qi, kj, scale, causal, rows, cols):
    s = scale * (qi @ kj.T)
    if causal:
        s = np.where(cols[None, :] <= rows[:, None], s, -np.inf)
    return s


def _exp_rel(x, ref):
    """exp(x - ref) with exp(-inf - (-inf)) taken as 0 (nothing accumulated yet)."""
    with np.errstate(invalid="ignore"):
        out = np.exp(x - ref)
    return np.where(np.isneginf(ref), 0.0, out)


def fa2_forward(q, k, v, scale, causal, key_blocks, row_blocks=None):
    """FA2 order for one head ([P1] "FlashAttention 2 forward pass 알고리즘 분석";
    the outer/inner loop of the [P2] tiling pseudocode).

    q, k, v: float64 [N, d]. key_blocks / row_blocks: block sizes along the keys
    and the query rows. For each query block Q_i (outer loop), initialise
    m = -inf, l = 0, O~ = 0 ([P2] pseudocode), then for each key block j in
    order (inner loop):
        S = scale * Q_i K_j^T
        m_new = max(m_old, rowmax(S))
        P~ = exp(S - m_new)
        alpha = exp(m_old - m_new)
        l = alpha * l + rowsum(P~)
        O~ = alpha * O~ + P~ V_j
    and finally O_i = O~ / l, L_i = m + log(l) ([P1] FA2 epilogue equation).
    Returns (O [N, d], L [N])."""
    N, d = q.shape
    row_blocks = row_blocks or [N]
    O = np.zeros((N, d))
    L = np.zeros(N)
    for r0, r1 in split_rows(N, row_blocks):
        rows = np.arange(r0, r1)
        m = np.full(r1 - r0, -np.inf)
        l = np.zeros(r1 - r0)
        acc = np.zeros((r1 - r0, d))
        for c0, c1 in split_rows(N, key_blocks):
            cols = np.arange(c0, c1)
            S = _scores(q[r0:r1], k[c0:c1], scale, causal, rows, cols)
            m_new = np.maximum(m, S.max(axis=1))
            P = _exp_rel(S, m_new[:, None])
            alpha = _exp_rel(m, m_new)
            l = alpha * l + P.sum(axis=1)
            acc = alpha[:, None] * acc + P @ v[c0:c1]
            m = m_new
        O[r0:r1] = acc / l[:, None]
        L[r0:r1] = m + np.log(l)
    return O, L


def fa1_forward(q, k, v, scale, causal, key_blocks, row_blocks=None):
    """FA1 order for one head ([P1] "FlashAttention 1 forward pass 알고리즘 분석").

    Outer loop over key blocks K_j, V_j; inner loop over query blocks Q_i, whose
    normalised O_i and statistics m_i, l_i are read and written back every time
    (the HBM round trip the page describes, here plain arrays). Per block:
        S = scale * Q_i K_j^T
        m~ = rowmax(S), P~ = exp(S - m~), l~ = rowsum(P~)
        m_new = max(m_i, m~), alpha = exp(m_i - m_new), beta = exp(m~ - m_new)
        l_new = alpha * l_i + beta * l~
        O_i <- diag(l_new)^-1 (diag(l_i) alpha O_i + beta P~ V_j)
    L = m + log(l) is formed at the end for comparison with FA2.
    Returns (O [N, d], L [N])."""
    N, d = q.shape
    row_blocks = row_blocks or [N]
    O = np.zeros((N, d))
    m_all = np.full(N, -np.inf)
    l_all = np.zeros(N)
    for c0, c1 in split_rows(N, key_blocks):
        cols = np.arange(c0, c1)
        for r0, r1 in split_rows(N, row_blocks):
            rows = np.arange(r0, r1)
            S = _scores(q[r0:r1], k[c0:c1], scale, causal, rows, cols)
            m_t = S.max(axis=1)
            P = _exp_rel(S, m_t[:, None])
            l_t = P.sum(axis=1)
            m_i, l_i, O_i = m_all[r0:r1], l_all[r0:r1], O[r0:r1]
            m_new = np.maximum(m_i, m_t)
            alpha = _exp_rel(m_i, m_new)
            beta = _exp_rel(m_t, m_new)
            l_new = alpha * l_i + beta * l_t
            num = (l_i * alpha)[:, None] * O_i + beta[:, None] * (P @ v[c0:c1])
            with np.errstate(invalid="ignore", divide="ignore"):
                O_new = np.where(l_new[:, None] > 0, num / l_new[:, None], 0.0)
            O[r0:r1] = O_new
            m_all[r0:r1] = m_new
            l_all[r0:r1] = l_new
    return O, m_all + np.log(l_all)
