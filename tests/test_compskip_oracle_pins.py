"""Pins of the layer-stack oracle (GDPA + HSP pooling + self-attention per layer,
with the CompSkip schedule; Kunlun paper summary, sections 2.1-2.3; Telegram
review, layer steps 1-5) against torch float64 autograd of an independent torch
implementation: SiLU FFN products per sample and head for GDPA, torch SDPA with
the seeds as queries for the pooling and with an explicit causal band mask for
the self-attention, and autograd for every gradient."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import gdpa_inputs as gi
from oracle import compskip_oracle as cs

H, D, N, C, M, W = 2, 8, 4, 6, 3, 3


def torch_stack(inp, schedule):
    """The layer stack written with torch library calls; returns (X_L, Z, grads)."""
    off = inp.offsets.numpy()
    B = len(off) - 1
    x0 = inp.x0.double().clone().requires_grad_()
    ctx = inp.ctx.double()
    wk = [w.double().clone().requires_grad_() for w in inp.w_k]
    wv = [w.double().clone().requires_grad_() for w in inp.w_v]
    sd = [s.double().clone().requires_grad_() for s in inp.seeds]
    x = x0
    zs = {}
    for l in range(len(wk)):
        # the schedule, from the pages: every op in every layer, or even layers
        # GDPA + pooling and odd layers self-attention only
        full = schedule == "full"
        run_g = full or l % 2 == 0
        run_s = full or l % 2 == 1
        if run_g:
            K = (ctx @ wk[l].T).reshape(B, N, H, D)
            V = (ctx @ wv[l].T).reshape(B, N, H, D)
            parts = []
            for b in range(B):
                xb = x[off[b]:off[b + 1]]                                  # [L, H, D]
                s_ = torch.einsum("lhd,nhd->hln", xb, K[b])
                parts.append(torch.einsum("hln,nhd->lhd", F.silu(s_), V[b]))
            x = x + torch.cat(parts, 0)
        xm = x
        if run_g:  # pooling runs with the PFFN
            zb = []
            for b in range(B):
                xb = xm[off[b]:off[b + 1]].transpose(0, 1)               # [H, L, D]
                if xb.shape[1] == 0:
                    zb.append(torch.zeros((M, H, D), dtype=torch.float64))
                    continue
                q = sd[l].transpose(0, 1)                                  # [H, M, D]
                zb.append(F.scaled_dot_product_attention(q, xb, xb, scale=1 / math.sqrt(D)).transpose(0, 1))
            zs[l] = torch.stack(zb, 0)
        if run_s:
            parts = []
            for b in range(B):
                L = off[b + 1] - off[b]
                xb = xm[off[b]:off[b + 1]].transpose(0, 1)
                i = torch.arange(L)[:, None]
                j = torch.arange(L)[None, :]
                band = (j <= i) & (j > i - W)
                o = F.scaled_dot_product_attention(xb, xb, xb, attn_mask=band, scale=1 / math.sqrt(D))
                parts.append(o.transpose(0, 1))
            x = xm + torch.cat(parts, 0)
    loss = (x * inp.dx.double()).sum() + sum((zs[l] * inp.dz[l].double()).sum() for l in zs)
    loss.backward()
    return (x.detach().numpy(), {l: z.detach().numpy() for l, z in zs.items()}, x0.grad.numpy(),
            {l: w.grad.numpy() for l, w in enumerate(wk) if w.grad is not None},
            {l: w.grad.numpy() for l, w in enumerate(wv) if w.grad is not None},
            {l: t.grad.numpy() for l, t in enumerate(sd) if t.grad is not None})


def rel(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


@pytest.mark.parametrize("schedule", cs.SCHEDULES)
def test_layer_stack_matches_torch_autograd(schedule):
    inp = gi.make_layer_stack_inputs(("explicit", [5, 0, 9, 4]), 4, H, D, N, C, layers=4, m=M, seed=3)
    recs, xl, zs = cs.forward(inp.x0, inp.offsets, inp.ctx, inp.w_k, inp.w_v, inp.seeds, H, N, W, schedule)
    dz = {l: inp.dz[l] for l in zs}
    dx0, dwk, dwv, dsd = cs.backward(recs, inp.offsets, inp.ctx, inp.w_k, inp.w_v, inp.seeds, H, N, W, schedule,
                                     inp.dx, dz)
    t_x, t_z, t_dx, t_wk, t_wv, t_sd = torch_stack(inp, schedule)
    assert rel(xl, t_x) <= 1e-12
    assert set(zs) == set(t_z) and all(rel(zs[l], t_z[l]) <= 1e-12 for l in zs)
    assert rel(dx0, t_dx) <= 1e-11
    assert set(dwk) == set(t_wk) and all(rel(dwk[l], t_wk[l]) <= 1e-11 for l in dwk)
    assert all(rel(dwv[l], t_wv[l]) <= 1e-11 for l in dwv)
    assert set(dsd) == set(t_sd) and all(rel(dsd[l], t_sd[l]) <= 1e-11 for l in dsd)


def test_compskip_layers_run_the_documented_ops():
    assert [cs.layer_ops("compskip", l) for l in range(4)] == [(True, True, False), (False, False, True)] * 2
    assert all(cs.layer_ops("full", l) == (True, True, True) for l in range(4))


def test_flop_accounting():
    lengths = [1000, 3000, 0, 500]
    full = cs.flops(lengths, 8, 128, 256, 512, 32, 512, 4, "full")
    skip = cs.flops(lengths, 8, 128, 256, 512, 32, 512, 4, "compskip")
    # CompSkip runs half the GDPA / pooling layers and half the self-attention layers.
    for k in ("gdpa", "weightgen", "hsp", "sa"):
        assert skip[k] == pytest.approx(full[k] / 2)
    pairs = sum(min(L, 512) * (min(L, 512) + 1) // 2 + (L - min(L, 512)) * 512 for L in lengths)
    assert full["sa"] == 4 * 12.0 * 8 * 128 * pairs
