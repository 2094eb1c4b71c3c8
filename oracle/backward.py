"""Plain float64 gradients of attention: the reference for the backward kernels.

TEST INFRASTRUCTURE ONLY (see the package docstring); the product path never
uses this module.

The pages describe the backward pass only by what it keeps and recomputes: the
forward stores the per-row logsumexp L instead of P, and the backward rebuilds P
block by block from S and L, since exp(S_ij - L_i) = P_ij ([P1] FA2 section,
the LSE identity; [P2] "FlashAttention: SRAM tiling으로 O(N²) HBM을 우회하다",
the activation-memory paragraph; [P3] "계산을 다시 하는 편이 싸다는 역설"). The
gradients themselves are not printed on the pages; they are the derivative of
the forward definition (the same formula as ``oracle.attention``), written out
with the chain rule. For the loss sum(O * dO), per batch b and head h:

    S   = scale * Q K^T, masked entries -inf      (forward definition)
    P   = softmax over the allowed keys of each row
    dV  = P^T dO
    dP  = dO V^T
    dS  = P * (dP - rowsum(P * dP))              (softmax Jacobian, row by row)
    dQ  = scale * dS K
    dK  = scale * dS^T Q

rowsum(P * dP) is the plain form of the softmax Jacobian; it equals
rowsum(dO * O), which the kernels use, so the two sides compute it differently.
L only enters through P here (its own gradient is not part of this pass).
"""
from __future__ import annotations

import numpy as np

__all__ = ["attention_backward"]


def _head_backward(q, k, v, do, scale, causal):
    n = q.shape[0]
    s = scale * (q @ k.T)
    if causal:
        allowed = np.arange(n)[None, :] <= np.arange(n)[:, None]
        s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return scale * (ds @ k), scale * (ds.T @ q), dv


def attention_backward(q, k, v, do, scale, causal):
    """dQ, dK, dV [B, H, N, d] (float64) of sum(O * dO) with O the attention output."""
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    B, H = q.shape[:2]
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = _head_backward(q[b, h], k[b, h], v[b, h],
                                                         do[b, h], scale, causal)
    return dq, dk, dv
