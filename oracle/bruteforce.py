"""Pure-Python attention for tiny inputs — TEST INFRASTRUCTURE ONLY.

An independent second formulation of the same definition, used to pin the
numpy oracle: it applies the softmax definition of [P1] "왜 필요한가"
literally, P_ij = exp(S_ij) / sum_j' exp(S_ij'), with no max shift, and sums
with ``math.fsum`` (exactly rounded sums). L_i is the log of that denominator.
It is only meant for small inputs with moderate scores, where exp cannot
overflow.
"""
from __future__ import annotations

import math

__all__ = ["attention_bruteforce"]


def attention_bruteforce(q, k, v, scale, causal):
    """q, k, v: nested sequences [B][H][N][d]. Returns (O, L) as nested lists."""
    O, L = [], []
    for qb, kb, vb in zip(q, k, v):
        Ob, Lb = [], []
        for qh, kh, vh in zip(qb, kb, vb):
            n = len(kh)
            d = len(vh[0]) if n else 0
            Oh, Lh = [], []
            for i, qi in enumerate(qh):
                keys = range(i + 1) if causal else range(n)
                w = [math.exp(scale * math.fsum(float(a) * float(b) for a, b in zip(qi, kh[j])))
                     for j in keys]
                denom = math.fsum(w)
                Oh.append([math.fsum(w[t] * float(vh[j][c]) for t, j in enumerate(keys)) / denom
                           for c in range(d)])
                Lh.append(math.log(denom))
            Ob.append(Oh)
            Lb.append(Lh)
        O.append(Ob)
        L.append(Lb)
    return O, L
