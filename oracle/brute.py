"""Scalar brute-force GDPA for tiny inputs (pure Python, no numpy, no BLAS).

TEST INFRASTRUCTURE ONLY (see gdpa_oracle.py).  This is a second, independent
spelling of the same definition, with explicit index loops and math.exp, used to
pin the vectorised oracle on tiny jagged batches (lengths including 0).

Definition (Kunlun paper summary, section 2.2, GDPA bullet): for every token t of
sample b and head h, s_j = scale * sum_e Q[t,h,e] K[b,j,h,e]; p = phi(s) over the
sample's n rows (a row softmax, or an elementwise SiLU, ReLU, GELU or identity);
O[t,h,e] = sum_j p_j V[b,j,h,e].
"""
from __future__ import annotations

import math


def _sigmoid(x: float) -> float:
    if x >= 0:
        return 1.0 / (1.0 + math.exp(-x))
    e = math.exp(x)
    return e / (1.0 + e)


def brute_forward(q, offsets, k, v, phi, scale):
    """q: nested lists [T][H][d]; k, v: [B][n][H][d]; offsets: list of B+1 ints.

    Returns (O as nested lists [T][H][d], lse [T][H] or None).
    """
    B = len(offsets) - 1
    T = offsets[-1]
    H = len(q[0]) if T else len(k[0][0])
    d = len(k[0][0][0])
    n = len(k[0])
    o = [[[0.0] * d for _ in range(H)] for _ in range(T)]
    lse = [[0.0] * H for _ in range(T)] if phi == "softmax" else None
    for b in range(B):
        for t in range(offsets[b], offsets[b + 1]):
            for h in range(H):
                s = []
                for j in range(n):
                    acc = 0.0
                    for e in range(d):
                        acc += q[t][h][e] * k[b][j][h][e]
                    s.append(scale * acc)
                if phi == "softmax":
                    m = max(s)
                    w = [math.exp(x - m) for x in s]
                    z = sum(w)
                    p = [x / z for x in w]
                    lse[t][h] = m + math.log(z)
                elif phi == "silu":
                    p = [x * _sigmoid(x) for x in s]
                elif phi == "relu":
                    p = [x if x > 0 else 0.0 for x in s]
                elif phi == "gelu":
                    p = [0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0))) for x in s]
                elif phi == "identity":
                    p = list(s)
                else:
                    raise ValueError(phi)
                for e in range(d):
                    acc = 0.0
                    for j in range(n):
                        acc += p[j] * v[b][j][h][e]
                    o[t][h][e] = acc
    return o, lse


def brute_swa_forward(q, offsets, k, v, window, scale):
    """Sliding-window self-attention (token i of a sample attends to its tokens j with
    i - window < j <= i), scalar loops; q, k, v: nested lists [T][H][d].
    Returns (O [T][H][d], lse [T][H])."""
    T = offsets[-1]
    H = len(q[0]) if T else 0
    d = len(q[0][0]) if T else 0
    o = [[[0.0] * d for _ in range(H)] for _ in range(T)]
    lse = [[0.0] * H for _ in range(T)]
    for b in range(len(offsets) - 1):
        for t in range(offsets[b], offsets[b + 1]):
            lo = max(offsets[b], t - window + 1)
            for h in range(H):
                s = []
                for u in range(lo, t + 1):
                    acc = 0.0
                    for e in range(d):
                        acc += q[t][h][e] * k[u][h][e]
                    s.append(scale * acc)
                m = max(s)
                wts = [math.exp(x - m) for x in s]
                z = sum(wts)
                lse[t][h] = m + math.log(z)
                for e in range(d):
                    acc = 0.0
                    for idx, u in enumerate(range(lo, t + 1)):
                        acc += wts[idx] / z * v[u][h][e]
                    o[t][h][e] = acc
    return o, lse
