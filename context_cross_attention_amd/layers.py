"""The Kunlun layer stack with the CompSkip schedule, driven through the C ABI.

A layer (Telegram review of the Kunlun paper, layer steps 1-5; paper summary,
sections 2.1 and 2.2) generates K, V from the context features, applies the
personalised FFN as GDPA with the tokens as queries, pools the sequence with
learned seeds (HSP) into summaries for the global interaction, and runs
self-attention over the context-enriched sequence:

    GDPA:  X' = X + GDPA_silu(X; C W_K^l, C W_V^l)
    HSP:   Z_l = Pool(Seeds_l; K = X', V = X')
    SA:    X'' = X' + SWA_w(X', X', X')

CompSkip (paper summary, section 2.3) alternates: even layers skip the
self-attention and compute fresh summaries, odd layers skip the pooling and the
PFFN.  The projections of the self-attention and of the pooling are identities
(outside the ops); the global interaction that reads Z_l is another system, so
Z_l is an output with its own upstream gradient.

All buffers are allocated once; a step only sequences library calls on the
current stream (GDPA, seed pooling, sliding-window attention, weight
generation and the fused residual sum).
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional

import torch

from . import (add_bf16, bwd, fwd, make_problem, pma_bwd, pma_fwd, pma_workspace_bytes, swa_block_bwd,
               swa_block_fwd, swa_workspace_bytes, weightgen_bwd_w, weightgen_fwd, workspace_bytes)

SCHEDULES = ("full", "compskip")


def layer_ops(schedule: str, l: int):
    """(run GDPA, run HSP, run SA) for layer l."""
    if schedule == "full":
        return True, True, True
    if schedule == "compskip":
        return (True, True, False) if l % 2 == 0 else (False, False, True)
    raise ValueError(f"schedule must be one of {SCHEDULES}")


class KunlunLayers:
    def __init__(self, offsets: torch.Tensor, ctx: torch.Tensor, w_k: List[torch.Tensor],
                 w_v: List[torch.Tensor], seeds: List[torch.Tensor], heads: int, n_kv: int,
                 total_tokens: int, window: int, schedule: str = "compskip", phi: str = "silu"):
        if phi == "softmax":
            raise NotImplementedError("the PFFN uses an elementwise map (the FFN form)")
        dev = ctx.device
        self.offsets, self.ctx, self.w_k, self.w_v, self.seeds = offsets, ctx, w_k, w_v, seeds
        self.L = len(w_k)
        self.B, self.c = ctx.shape
        self.H, self.n, self.T, self.w = heads, n_kv, total_tokens, window
        self.d = w_k[0].shape[0] // (n_kv * heads)
        self.m = seeds[0].shape[0]
        self.schedule, self.phi = schedule, phi
        self.ops = [layer_ops(schedule, l) for l in range(self.L)]
        T, H, d, B, n, m = self.T, self.H, self.d, self.B, self.n, self.m
        bf = torch.bfloat16
        tok = lambda: torch.empty((T, H, d), dtype=bf, device=dev)
        # Per layer: input state, state after the PFFN (the pooled / attended one),
        # K and V, the self-attention output and LSE, the summaries and their LSE.
        self.x_in = [None] * self.L
        self.x_mid = [tok() if g else None for g, _, _ in self.ops]
        self.x_out = [tok() if s else None for _, _, s in self.ops]
        self.k = [torch.empty((B, n, H, d), dtype=bf, device=dev) if g else None for g, _, _ in self.ops]
        self.v = [torch.empty((B, n, H, d), dtype=bf, device=dev) if g else None for g, _, _ in self.ops]
        self.sa_o = [tok() if s else None for _, _, s in self.ops]
        self.sa_lse = [torch.empty((T, H), dtype=torch.float32, device=dev) if s else None for _, _, s in self.ops]
        self.z = [torch.empty((B, m, H, d), dtype=bf, device=dev) if h else None for _, h, _ in self.ops]
        self.z_lse = [torch.empty((B, m, H), dtype=torch.float32, device=dev) if h else None for _, h, _ in self.ops]
        # Backward: two gradient states, the pooling's dK + dV, GDPA's dK / dV.
        self.gx = [tok(), tok()]
        self.g2 = tok()
        self.dk = torch.empty((B, n, H, d), dtype=bf, device=dev)
        self.dv = torch.empty((B, n, H, d), dtype=bf, device=dev)
        self.dw_k = {l: torch.empty_like(w_k[l]) for l in range(self.L) if self.ops[l][0]}
        self.dw_v = {l: torch.empty_like(w_v[l]) for l in range(self.L) if self.ops[l][0]}
        self.dseeds = {l: torch.empty_like(seeds[l]) for l in range(self.L) if self.ops[l][1]}
        # One workspace, sized for the largest of the calls (shapes only are read).
        x_probe = self.gx[0]
        prob = make_problem(x_probe, offsets, self.dk, phi, None, 0)
        ws = max([workspace_bytes(prob, bw) for bw in (False, True)] +
                 [swa_workspace_bytes(x_probe, offsets, window, bw) for bw in (False, True)] +
                 [pma_workspace_bytes(seeds[0], offsets, x_probe, bw) for bw in (False, True)] + [1])
        self.ws = torch.empty(ws, dtype=torch.uint8, device=dev)

    def forward(self, x0: torch.Tensor, mark: Optional[Callable[[str, bool], None]] = None):
        """X_0 = x0 [T, H, d]; returns (X_L, {l: Z_l})."""
        mark = mark or (lambda name, start: None)
        x = x0.view(self.T, self.H, self.d)
        for l, (run_g, run_h, run_s) in enumerate(self.ops):
            self.x_in[l] = x
            if run_g:
                mark("weightgen_fwd", True)
                weightgen_fwd(self.ctx, self.w_k[l], out=self.k[l].view(self.B, -1))
                weightgen_fwd(self.ctx, self.w_v[l], out=self.v[l].view(self.B, -1))
                mark("weightgen_fwd", False)
                mark("gdpa_fwd", True)
                fwd(x, self.offsets, self.k[l], self.v[l], phi=self.phi, residual=x, out=self.x_mid[l],
                    workspace=self.ws)
                mark("gdpa_fwd", False)
                x = self.x_mid[l]
            if run_h:
                mark("hsp_fwd", True)
                pma_fwd(self.seeds[l], self.offsets, x, x, out=self.z[l], lse=self.z_lse[l], workspace=self.ws)
                mark("hsp_fwd", False)
            if run_s:
                mark("sa_fwd", True)
                swa_block_fwd(x, self.offsets, self.w, o=self.sa_o[l], y=self.x_out[l], lse=self.sa_lse[l],
                              workspace=self.ws)
                mark("sa_fwd", False)
                x = self.x_out[l]
        return x, {l: self.z[l] for l in range(self.L) if self.z[l] is not None}

    def backward(self, g: torch.Tensor, gz: Dict[int, torch.Tensor],
                 mark: Optional[Callable[[str, bool], None]] = None):
        """Upstream gradients g = dLoss/dX_L and gz[l] = dLoss/dZ_l; returns
        (dX_0, {l: dW_K^l}, {l: dW_V^l}, {l: dSeeds_l})."""
        mark = mark or (lambda name, start: None)
        src = g.view(self.T, self.H, self.d)
        flip = 0
        for l in reversed(range(self.L)):
            run_g, run_h, run_s = self.ops[l]
            xm = self.x_mid[l] if run_g else self.x_in[l]
            if run_s:  # X'' = X' + SWA(X', X', X'): dX' = dX'' + dQ + dK + dV
                mark("sa_bwd", True)
                dst = self.gx[flip]
                swa_block_bwd(xm, self.offsets, self.sa_o[l], self.sa_lse[l], src, self.w, dx=dst, workspace=self.ws)
                mark("sa_bwd", False)
                src, flip = dst, flip ^ 1
            if run_h:  # Z = Pool(Seeds; X', X')
                mark("hsp_bwd", True)
                pma_bwd(self.seeds[l], self.offsets, xm, xm, self.z[l], self.z_lse[l], gz[l],
                        d_seeds=self.dseeds[l], dk=self.g2, workspace=self.ws, kv_sum=True)
                dst = self.gx[flip]
                add_bf16(dst, src, self.g2)
                mark("hsp_bwd", False)
                src, flip = dst, flip ^ 1
            if run_g:  # X' = X + GDPA(X; K, V): dX = dX' + dQ
                dst = self.gx[flip]
                mark("gdpa_bwd", True)
                bwd(self.x_in[l], self.offsets, self.k[l], self.v[l], None, None, src, phi=self.phi, dq=dst,
                    residual=True, dk=self.dk, dv=self.dv, workspace=self.ws)
                mark("gdpa_bwd", False)
                mark("weightgen_bwd", True)
                weightgen_bwd_w(self.ctx, self.dk.view(self.B, -1), d_w=self.dw_k[l])
                weightgen_bwd_w(self.ctx, self.dv.view(self.B, -1), d_w=self.dw_v[l])
                mark("weightgen_bwd", False)
                src, flip = dst, flip ^ 1
        return src, self.dw_k, self.dw_v, self.dseeds
