"""Stacked residual GDPA layers with generated K/V, driven through the C ABI.

Each layer (Telegram review of the Kunlun paper, layer steps 1-2; paper summary
section 2.2, GDPA bullet: the personalised FFN becomes stable to stack, read here
as a plain residual with no normalisation):

    K_l = C W_K^l^T,  V_l = C W_V^l^T             (weight generation, W: [n*H*d, c])
    X_{l+1} = X_l + GDPA_phi(X_l; K_l, V_l)       (queries are the token states)

Backward of sum(X_L * G):
    dX_l = dX_{l+1} + dQ_l,   dW_K^l = dK_l^T C,   dW_V^l = dV_l^T C.

All buffers are allocated once; a step only sequences library calls on the
current stream.  With the row softmax the backward needs each layer's LSE; where it
also reads the un-summed output O_l for its row term (shapes outside the
one-work-group backward, see bwd_reads_o) the forward keeps O_l too (gdpa_fwd_block
writes O_l and X_l + O_l in one pass).  The elementwise maps need neither.
"""
from __future__ import annotations

from typing import Callable, List, Optional

import torch

from . import bwd, bwd_reads_o, fwd, fwd_block, make_problem, weightgen_bwd_w, weightgen_fwd, workspace_bytes


class StackedGdpa:
    def __init__(self, offsets: torch.Tensor, ctx: torch.Tensor, w_k: List[torch.Tensor],
                 w_v: List[torch.Tensor], heads: int, n_kv: int, total_tokens: int,
                 phi: str = "silu", scale: Optional[float] = None):
        dev = ctx.device
        self.offsets, self.ctx, self.w_k, self.w_v = offsets, ctx, w_k, w_v
        self.L = len(w_k)
        self.B, self.c = ctx.shape
        self.H, self.n = heads, n_kv
        self.d = w_k[0].shape[0] // (n_kv * heads)
        self.T = total_tokens
        self.phi, self.scale = phi, scale
        T, H, d, B, n = self.T, self.H, self.d, self.B, self.n
        bf = torch.bfloat16
        # x[0] is the caller's input (set by forward, not copied); x[1..L] are outputs.
        self.x = [None] + [torch.empty((T, H, d), dtype=bf, device=dev) for _ in range(self.L)]
        self.k = [torch.empty((B, n, H, d), dtype=bf, device=dev) for _ in range(self.L)]
        self.v = [torch.empty((B, n, H, d), dtype=bf, device=dev) for _ in range(self.L)]
        self.gx = [torch.empty((T, H, d), dtype=bf, device=dev) for _ in range(2)]
        self.dk = torch.empty((B, n, H, d), dtype=bf, device=dev)
        self.dv = torch.empty((B, n, H, d), dtype=bf, device=dev)
        self.dw_k = [torch.empty_like(w) for w in w_k]
        self.dw_v = [torch.empty_like(w) for w in w_v]
        softmax = phi == "softmax"
        keep_o = softmax and bwd_reads_o(bf, d, n)
        # softmax: each layer's LSE (and, where the backward reads it, its GDPA output).
        self.o = [torch.empty((T, H, d), dtype=bf, device=dev) for _ in range(self.L)] if keep_o else None
        self.lse = [torch.empty((T, H), dtype=torch.float32, device=dev) for _ in range(self.L)] if softmax else None
        probe_q = torch.empty((T, H, d), dtype=bf, device="meta")
        probe_k = torch.empty((B, n, H, d), dtype=bf, device="meta")
        prob = make_problem(probe_q, None, probe_k, phi, scale)
        self.ws_f = torch.empty(max(workspace_bytes(prob, False), 256), dtype=torch.uint8, device=dev)
        self.ws_b = torch.empty(max(workspace_bytes(prob, True), 256), dtype=torch.uint8, device=dev)

    def forward(self, x0: torch.Tensor, mark: Optional[Callable[[str, bool], None]] = None):
        """X_0 = x0 ([T, H*d] or [T, H, d]); returns X_L ([T, H, d])."""
        mark = mark or (lambda name, start: None)
        self.x[0] = x0.view(self.T, self.H, self.d)
        for l in range(self.L):
            mark("weightgen_fwd", True)
            weightgen_fwd(self.ctx, self.w_k[l], out=self.k[l].view(self.B, -1))
            weightgen_fwd(self.ctx, self.w_v[l], out=self.v[l].view(self.B, -1))
            mark("weightgen_fwd", False)
            mark("gdpa_fwd", True)
            if self.o is not None:
                fwd_block(self.x[l], self.offsets, self.k[l], self.v[l], phi=self.phi, scale=self.scale,
                          o=self.o[l], y=self.x[l + 1], lse=self.lse[l], workspace=self.ws_f)
            else:
                fwd(self.x[l], self.offsets, self.k[l], self.v[l], phi=self.phi, scale=self.scale,
                    residual=self.x[l], out=self.x[l + 1],
                    lse=self.lse[l] if self.lse is not None else None, workspace=self.ws_f)
            mark("gdpa_fwd", False)
        return self.x[self.L]

    def backward(self, g: torch.Tensor, mark: Optional[Callable[[str, bool], None]] = None):
        """Upstream gradient g = dL/dX_L; returns (dX_0, [dW_K], [dW_V])."""
        mark = mark or (lambda name, start: None)
        g = g.view(self.T, self.H, self.d)
        src = g
        for i, l in enumerate(reversed(range(self.L))):
            dst = self.gx[i % 2]
            mark("gdpa_bwd", True)
            o_l = self.o[l] if self.o is not None else None
            lse_l = self.lse[l] if self.lse is not None else None
            bwd(self.x[l], self.offsets, self.k[l], self.v[l], o_l, lse_l, src, phi=self.phi,
                scale=self.scale, dq=dst, residual=True, dk=self.dk, dv=self.dv,
                workspace=self.ws_b)
            mark("gdpa_bwd", False)
            mark("weightgen_bwd", True)
            weightgen_bwd_w(self.ctx, self.dk.view(self.B, -1), d_w=self.dw_k[l])
            weightgen_bwd_w(self.ctx, self.dv.view(self.B, -1), d_w=self.dw_v[l])
            mark("weightgen_bwd", False)
            src = dst
        return src, self.dw_k, self.dw_v
