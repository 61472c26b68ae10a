"""fp64 CPU oracle for seed pooling attention over a jagged batch.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

What it computes: the Kunlun paper summary (section 2.1, interaction block, and
section 2.2, Hierarchical Seed Pooling bullet) summarises long sequences with
learnable seed queries that attend over the sequence, as Pooling by Multihead
Attention does, before the hierarchical compression (SumKronLinear, given no
formula on the pages and not computed here); the Telegram review (layer step 3)
describes HSP as the replacement of PMA that carries the history to the context
features.  The attention core: for sample b (rows offsets[b] .. offsets[b+1]-1
of K, V [T,H,d]), seed s and head h,

    S[s, j]    = scale * < Seeds[s,h,:], K[j,h,:] >       j over the sample's tokens
    O[b,s,h,:] = sum_j softmax_j(S[s, :]) V[j,h,:]

Readings: the seeds [m,H,d] are shared by all samples; row softmax over the
sample's tokens with scale 1/sqrt(d) by default; no mask; an empty sample has
no tokens to pool, so its output and its share of every gradient are zero.
The backward is that of softmax attention with the seeds as queries; the seed
gradient sums over every sample.

Plain float64 numpy per sample and head; a matrix product is the only library
step.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

from oracle.gdpa_oracle import as_f64, row_softmax


def _check(seeds, offsets, k, v):
    if k.shape != v.shape or k.ndim != 3:
        raise ValueError("K and V must be [T, H, d]")
    m, H, d = seeds.shape
    if k.shape[1:] != (H, d):
        raise ValueError("seeds must be [m, H, d] with the heads and width of K")
    T = k.shape[0]
    if offsets[0] != 0 or offsets[-1] != T or np.any(np.diff(offsets) < 0):
        raise ValueError("offsets must be non-decreasing from 0 to T")
    return m, H, d, len(offsets) - 1


def pma_forward(seeds, offsets, k, v, scale: Optional[float] = None,
                samples: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """(O [B,m,H,d], LSE [B,m,H]) in float64; zeros and -inf for an empty sample.  With
    `samples`, only those samples are computed (the others stay NaN)."""
    seeds, k, v = as_f64(seeds), as_f64(k), as_f64(v)
    offsets = np.asarray(as_f64(offsets), dtype=np.int64)
    m, H, d, B = _check(seeds, offsets, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((B, m, H, d))
    lse = np.full((B, m, H), -np.inf)
    if samples is not None:
        o[:] = np.nan
        lse[:] = np.nan
    for b in (range(B) if samples is None else samples):
        r = slice(int(offsets[b]), int(offsets[b + 1]))
        if r.stop == r.start:
            o[b] = 0.0
            lse[b] = -np.inf
            continue
        for h in range(H):
            p, l = row_softmax(scale * (seeds[:, h, :] @ k[r, h, :].T))    # [m, L]
            o[b, :, h, :] = p @ v[r, h, :]
            lse[b, :, h] = l
    return o, lse


def pma_backward(seeds, offsets, k, v, do, scale: Optional[float] = None,
                 samples: Optional[Sequence[int]] = None):
    """Gradients of sum(O * dO): (dSeeds [m,H,d] summed over samples, dK, dV [T,H,d]).
    With `samples`, only those samples contribute (dSeeds is their sum; the other
    samples' dK, dV rows stay NaN).

    Per sample and head: dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dO * O)),
    dSeeds += scale dS K, dK = scale dS^T Seeds."""
    seeds, k, v, do = as_f64(seeds), as_f64(k), as_f64(v), as_f64(do)
    offsets = np.asarray(as_f64(offsets), dtype=np.int64)
    m, H, d, B = _check(seeds, offsets, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dseeds = np.zeros((m, H, d))
    dk = np.zeros(k.shape) if samples is None else np.full(k.shape, np.nan)
    dv = np.zeros(v.shape) if samples is None else np.full(v.shape, np.nan)
    for b in (range(B) if samples is None else samples):
        r = slice(int(offsets[b]), int(offsets[b + 1]))
        if r.stop == r.start:
            continue
        for h in range(H):
            kb, vb, sd, g = k[r, h, :], v[r, h, :], seeds[:, h, :], do[b, :, h, :]
            p, _ = row_softmax(scale * (sd @ kb.T))
            o = p @ vb
            ds = p * ((g @ vb.T) - (g * o).sum(axis=-1, keepdims=True))
            dseeds[:, h, :] += scale * (ds @ kb)
            dk[r, h, :] = scale * (ds.T @ sd)
            dv[r, h, :] = p.T @ g
    return dseeds, dk, dv
