"""Pins of the oracle's biased form O = phi(scale X K^T + b_s) V + b_o (the two
biases of a two-layer FFN: one per hidden unit, i.e. per context row, and one per
output column; per sample and head like K and V): the elementwise maps equal a
two-layer FFN built with torch.nn.functional.linear and its bias arguments; the
softmax map equals torch SDPA with the score bias as an additive float mask;
torch autograd for every gradient, including both bias gradients; jagged
contexts; b = 0 reduces to the unbiased oracle."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import gdpa_inputs as gi
from oracle import gdpa_oracle as orc

ACT = {"silu": F.silu, "relu": F.relu, "gelu": F.gelu, "identity": lambda t: t}


def rel(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


def problem(seed, lengths, counts, H=2, d=8):
    inp = gi.make_jagged_kv_inputs(("explicit", list(lengths)), ("explicit", list(counts)), len(lengths), H, d,
                                   seed=seed, sharp=True, dtype="f32")
    rng = np.random.default_rng(seed + 100)
    sb = rng.standard_normal((inp.k.shape[0], H))
    ob = rng.standard_normal((len(lengths), H, d))
    return inp, sb, ob


def torch_ref(inp, sb, ob, phi, scale):
    """Per sample and head: F.linear FFN (elementwise maps) or SDPA with a float mask."""
    q = torch.from_numpy(inp.q.double().numpy()).requires_grad_()
    k = torch.from_numpy(inp.k.double().numpy()).requires_grad_()
    v = torch.from_numpy(inp.v.double().numpy()).requires_grad_()
    tsb = torch.from_numpy(sb).requires_grad_()
    tob = torch.from_numpy(ob).requires_grad_()
    off, ko = inp.offsets.numpy(), inp.kv_offsets.numpy()
    B, H = len(off) - 1, q.shape[1]
    outs = [None] * len(q)
    rows = []
    for b in range(B):
        r, c = slice(off[b], off[b + 1]), slice(ko[b], ko[b + 1])
        heads = []
        for h in range(H):
            x, kb, vb, bs = q[r, h], k[c, h], v[c, h], tsb[c, h]
            if phi == "softmax":
                o = F.scaled_dot_product_attention(x[None], kb[None], vb[None], attn_mask=bs[None, None, :].expand(1, x.shape[0], -1),
                                                   scale=scale)[0]
            else:
                hid = ACT[phi](F.linear(x * scale, kb, bs))     # [L, n]: scale x K^T + b_s
                o = hid @ vb
            heads.append(o + tob[b, h][None, :])
        rows.append(torch.stack(heads, 1))
    o = torch.cat(rows, 0)
    g = torch.from_numpy(np.random.default_rng(7).standard_normal(o.shape))
    (o * g).sum().backward()
    return o.detach().numpy(), g.numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy(), tsb.grad.numpy(), tob.grad.numpy()


@pytest.mark.parametrize("phi", orc.PHIS)
def test_biased_forward_and_backward_match_torch(phi):
    inp, sb, ob = problem(1, (5, 0, 9, 3), (4, 2, 7, 1))
    scale = orc.default_scale(phi, 8) if phi == "softmax" else 0.7
    o, _ = orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, phi, scale, kv_offsets=inp.kv_offsets,
                            score_bias=sb, out_bias=ob)
    t_o, g, t_dq, t_dk, t_dv, t_dsb, t_dob = torch_ref(inp, sb, ob, phi, scale)
    assert rel(o, t_o) <= 1e-12
    dq, dk, dv, dsb, dob = orc.gdpa_backward(inp.q, inp.offsets, inp.k, inp.v, g, phi, scale,
                                             kv_offsets=inp.kv_offsets, score_bias=sb, bias_grads=True)
    for a, b in ((dq, t_dq), (dk, t_dk), (dv, t_dv), (dsb, t_dsb), (dob, t_dob)):
        assert rel(a, b) <= 1e-11


def test_zero_biases_reduce_to_unbiased():
    inp, sb, ob = problem(2, (6, 4), (3, 5))
    for phi in ("softmax", "silu"):
        o0, l0 = orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, phi, kv_offsets=inp.kv_offsets)
        o1, l1 = orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, phi, kv_offsets=inp.kv_offsets,
                                  score_bias=np.zeros_like(sb), out_bias=np.zeros_like(ob))
        assert np.array_equal(o0, o1)


def test_dense_layout_biases():
    # The dense [B,n,H] score-bias layout gives the same result as the jagged one with equal counts.
    inp, sb, ob = problem(3, (6, 4, 2), (3, 3, 3))
    kd, vd = inp.k.view(3, 3, 2, 8), inp.v.view(3, 3, 2, 8)
    oj, _ = orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, "gelu", kv_offsets=inp.kv_offsets,
                             score_bias=sb, out_bias=ob)
    od, _ = orc.gdpa_forward(inp.q, inp.offsets, kd, vd, "gelu", score_bias=sb.reshape(3, 3, 2), out_bias=ob)
    assert np.array_equal(oj, od)
    gj = orc.gdpa_backward(inp.q, inp.offsets, inp.k, inp.v, inp.do, "gelu", kv_offsets=inp.kv_offsets,
                           score_bias=sb, bias_grads=True)
    gd = orc.gdpa_backward(inp.q, inp.offsets, kd, vd, inp.do, "gelu", score_bias=sb.reshape(3, 3, 2),
                           bias_grads=True)
    assert np.array_equal(gj[3], gd[3].reshape(9, 2)) and np.array_equal(gj[4], gd[4])
