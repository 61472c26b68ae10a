"""fp64 CPU oracle for the Kunlun layer stack with Computation Skip (CompSkip).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

What it computes.  A Kunlun layer (Telegram review, layer steps 1-5; Kunlun
paper summary, sections 2.1 and 2.2) generates K, V from the context features,
applies the personalised FFN as GDPA with the tokens as queries, pools the
sequence with learned seeds (HSP), hands the summaries to the global
interaction, and runs self-attention over the context-enriched sequence.
CompSkip (paper summary, section 2.3, CompSkip bullet) alternates: even layers
skip the self-attention and compute fresh HSP summaries, odd layers skip HSP
and the PFFN and compute the self-attention.

    GDPA:  X' = X + GDPA_phi(X; C W_K^l, C W_V^l)
    HSP:   Z_l = Pool(Seeds_l; K = X', V = X')                 (an output of the layer)
    SA:    X'' = X' + SWA_w(Q = X', K = X', V = X')

Schedules: "full" runs all three in every layer; "compskip" runs GDPA and HSP
in even layers and SA in odd layers.  Readings (the pages give no formula): the
projections of the self-attention and of the pooling are identities (outside
the ops, as for the ops themselves); the global interaction that consumes Z_l
(Wukong) is another system, so Z_l is an output of the stack with its own
upstream gradient; the residuals are plain sums.

The arithmetic is the pinned single-op oracles composed: gdpa_oracle,
pma_oracle and swa_oracle; the only new steps are the residual sums and the
sums of gradient contributions where one tensor feeds several inputs.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from oracle import gdpa_oracle as g
from oracle import pma_oracle as p
from oracle import swa_oracle as s

SCHEDULES = ("full", "compskip")


def layer_ops(schedule: str, l: int):
    """(run GDPA, run HSP, run SA) for layer l of a schedule."""
    if schedule == "full":
        return True, True, True
    if schedule == "compskip":
        return (True, True, False) if l % 2 == 0 else (False, False, True)
    raise ValueError(schedule)


def forward(x0, offsets, ctx, w_k: List, w_v: List, seeds: List, heads: int, n: int, window: int,
            schedule: str, phi: str = "silu"):
    """Returns (per-layer records, X_L [T,H,d], {l: Z_l [B,m,H,d]}).  x0: [T,H,d]."""
    x = g.as_f64(x0)
    T, H, d = x.shape
    recs, zs = [], {}
    for l in range(len(w_k)):
        run_g, run_h, run_s = layer_ops(schedule, l)
        rec = {"x_in": x}
        if run_g:
            kl = g.weight_generation(ctx, w_k[l], n, H, d)
            vl = g.weight_generation(ctx, w_v[l], n, H, d)
            o, _ = g.gdpa_forward(x, offsets, kl, vl, phi)
            x = x + o
        rec["x_mid"] = x
        if run_h:
            zs[l], _ = p.pma_forward(seeds[l], offsets, x, x)
        if run_s:
            o, _ = s.swa_forward(x, offsets, x, x, window)
            x = x + o
        recs.append(rec)
    return recs, x, zs


def backward(recs, offsets, ctx, w_k: List, w_v: List, seeds: List, heads: int, n: int, window: int,
             schedule: str, dx_out, dz: Dict[int, np.ndarray], phi: str = "silu"):
    """Backward for the loss sum(X_L * dx_out) + sum_l sum(Z_l * dz[l]).

    Returns (dX_0, {l: dW_K^l}, {l: dW_V^l}, {l: dSeeds_l})."""
    ctx = g.as_f64(ctx)
    dx = g.as_f64(dx_out)
    T, H, d = dx.shape
    B = ctx.shape[0]
    dwk, dwv, dseeds = {}, {}, {}
    for l in reversed(range(len(w_k))):
        run_g, run_h, run_s = layer_ops(schedule, l)
        xm, xi = recs[l]["x_mid"], recs[l]["x_in"]
        if run_s:  # X'' = X' + SWA(X', X', X'): all three inputs are X'
            gq, gk, gv = s.swa_backward(xm, offsets, xm, xm, dx, window)
            dx = dx + gq + gk + gv
        if run_h:  # Z = Pool(Seeds; X', X')
            gs, gk, gv = p.pma_backward(seeds[l], offsets, xm, xm, dz[l])
            dseeds[l] = gs
            dx = dx + gk + gv
        if run_g:  # X' = X + GDPA(X; C W_K^T, C W_V^T)
            kl = g.weight_generation(ctx, w_k[l], n, H, d)
            vl = g.weight_generation(ctx, w_v[l], n, H, d)
            gq, gk, gv = g.gdpa_backward(xi, offsets, kl, vl, dx, phi)
            dwk[l] = g.weight_gradient(ctx, gk.reshape(B, -1))
            dwv[l] = g.weight_gradient(ctx, gv.reshape(B, -1))
            dx = dx + gq
    return dx, dwk, dwv, dseeds


def flops(lengths: Sequence[int], heads: int, d: int, n: int, ctx_dim: int, m: int, window: int,
          layers: int, schedule: str) -> Dict[str, float]:
    """Algorithmic FLOPs of one forward + backward step, per op kind.

    GDPA 12 T H n d (4 forward, 8 backward); weight generation 2 x (forward and
    weight-gradient GEMMs) of 2 B (n H d) c each; pooling 14 T H m d (4 + 10);
    sliding window 12 H d per in-window (token, key) pair."""
    T = float(sum(lengths))
    B = len(lengths)
    pairs = 0
    for L in lengths:
        L = int(L)
        k = min(L, window)
        pairs += k * (k + 1) // 2 + (L - k) * window
    out = {"gdpa": 0.0, "weightgen": 0.0, "hsp": 0.0, "sa": 0.0}
    for l in range(layers):
        run_g, run_h, run_s = layer_ops(schedule, l)
        if run_g:
            out["gdpa"] += 12.0 * T * heads * n * d
            out["weightgen"] += 4 * 2.0 * B * (n * heads * d) * ctx_dim
        if run_h:
            out["hsp"] += 14.0 * T * heads * m * d
        if run_s:
            out["sa"] += 12.0 * heads * d * pairs
    out["total"] = sum(out.values())
    return out
