"""fp64 CPU oracle for sliding-window self-attention over a jagged batch.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

What it computes: the Kunlun paper summary (section 2.2, "Sliding Window
Attention" bullet) restricts the sequence's self-attention to local windows,
so that its cost falls from O(T^2) to O(T w) and each event looks at the most
recent interactions; the Telegram review lists the block as standard
self-attention over the context-enriched sequence (layer step 5) and names w,
the window size, among the per-sequence hyper-parameters of event-level
personalisation.  For a jagged batch (sample b owns rows offsets[b] ..
offsets[b+1]-1 of Q, K, V [T,H,d]) and head h, with i, j token positions inside
the sample:

    S[i, j] = scale * < Q[i,h,:], K[j,h,:] >      for  i - w < j <= i
    P[i, :] = softmax over those j                  (every other j is excluded)
    O[i,h,:] = sum_j P[i, j] V[j,h,:]

Readings taken (the pages give no formula): the window is causal and holds the
token itself and the w - 1 tokens before it in its own sample ("recent
interactions"); the score map is the row softmax of standard attention, scale
1/sqrt(d) by default; Q, K and V projections are outside the operation, as for
GDPA.  The backward is that of softmax attention restricted to the same pairs.

Plain float64 numpy per sample and head; a matrix product is the only library
step.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

from oracle.gdpa_oracle import as_f64


def band_mask(L: int, w: int) -> np.ndarray:
    """M[i, j] = True where token i attends to token j: i - w < j <= i."""
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    return (j <= i) & (j > i - w)


def swa_forward_bh(xq: np.ndarray, xk: np.ndarray, xv: np.ndarray, w: int,
                   scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """O and the natural-log LSE of one sample and head (xq, xk, xv: [L, d])."""
    L = xq.shape[0]
    s = scale * (xq @ xk.T)
    s = np.where(band_mask(L, w), s, -np.inf)
    m = s.max(axis=-1, keepdims=True)           # finite: j = i is always allowed
    e = np.exp(s - m)
    l = e.sum(axis=-1, keepdims=True)
    p = e / l
    return p @ xv, (m + np.log(l))[:, 0]


def swa_backward_bh(xq, xk, xv, do, w: int, scale: float):
    """Gradients of sum(O * dO) with respect to xq, xk, xv for one sample and head:
    dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dO * O)), dQ = scale dS K,
    dK = scale dS^T Q (P is zero outside the window)."""
    L = xq.shape[0]
    s = scale * (xq @ xk.T)
    s = np.where(band_mask(L, w), s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=-1, keepdims=True)
    o = p @ xv
    dp = do @ xv.T
    ds = p * (dp - (do * o).sum(axis=-1, keepdims=True))
    return scale * (ds @ xk), scale * (ds.T @ xq), p.T @ do


def _check(q, offsets, k, v, window):
    if q.shape != k.shape or q.shape != v.shape or q.ndim != 3:
        raise ValueError("Q, K and V must all be [T, H, d]")
    T = q.shape[0]
    if offsets[0] != 0 or offsets[-1] != T or np.any(np.diff(offsets) < 0):
        raise ValueError("offsets must be non-decreasing from 0 to T")
    if window < 1:
        raise ValueError("window must be at least 1")
    return q.shape


def swa_forward(q, offsets, k, v, window: int, scale: Optional[float] = None,
                samples: Optional[Sequence[int]] = None):
    """Jagged forward: (O [T,H,d], LSE [T,H]) in float64; with `samples`, only
    those samples' rows are computed (the rest stay NaN)."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    offsets = np.asarray(as_f64(offsets), dtype=np.int64)
    T, H, d = _check(q, offsets, k, v, window)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.full((T, H, d), np.nan)
    lse = np.full((T, H), np.nan)
    B = len(offsets) - 1
    for b in (range(B) if samples is None else samples):
        r = slice(int(offsets[b]), int(offsets[b + 1]))
        for h in range(H):
            if r.stop > r.start:
                o[r, h, :], lse[r, h] = swa_forward_bh(q[r, h, :], k[r, h, :], v[r, h, :], window, scale)
    return o, lse


def swa_backward(q, offsets, k, v, do, window: int, scale: Optional[float] = None,
                 samples: Optional[Sequence[int]] = None):
    """Jagged backward: (dQ, dK, dV), each [T,H,d] float64."""
    q, k, v, do = as_f64(q), as_f64(k), as_f64(v), as_f64(do)
    offsets = np.asarray(as_f64(offsets), dtype=np.int64)
    T, H, d = _check(q, offsets, k, v, window)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = (np.full((T, H, d), np.nan) for _ in range(3))
    B = len(offsets) - 1
    for b in (range(B) if samples is None else samples):
        r = slice(int(offsets[b]), int(offsets[b + 1]))
        for h in range(H):
            if r.stop > r.start:
                dq[r, h, :], dk[r, h, :], dv[r, h, :] = swa_backward_bh(
                    q[r, h, :], k[r, h, :], v[r, h, :], do[r, h, :], window, scale)
    return dq, dk, dv
