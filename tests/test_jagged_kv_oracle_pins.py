"""Pins of the oracle's jagged-context form (each sample owns its own number of
context rows; Kunlun paper summary, section 2.3, Event-Level Personalization
bullet, and the Telegram review's per-event n_tokens): the jagged batch equals
independent one-sample dense calls; for the elementwise maps it equals the dense
form with every context zero-padded to the longest (phi(0) = 0); for softmax
zero padding changes the result (a padded context is not the same op); torch
SDPA per sample; input validation."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import gdpa_inputs as gi
from oracle import gdpa_oracle as orc


def problem(seed, lengths, counts, H=2, d=8, sharp=True):
    return gi.make_jagged_kv_inputs(("explicit", list(lengths)), ("explicit", list(counts)), len(lengths),
                                    H, d, seed=seed, sharp=sharp, dtype="f32")


def rel(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


def padded(inp, n):
    """Dense [B,n,H,d] copies of the jagged K, V with zero rows past each sample's count."""
    B = len(inp.kv_counts)
    H, d = inp.k.shape[1:]
    kd = np.zeros((B, n, H, d))
    vd = np.zeros((B, n, H, d))
    ko = inp.kv_offsets.numpy()
    for b in range(B):
        c = ko[b + 1] - ko[b]
        kd[b, :c] = inp.k.numpy()[ko[b]:ko[b + 1]]
        vd[b, :c] = inp.v.numpy()[ko[b]:ko[b + 1]]
    return kd, vd


@pytest.mark.parametrize("phi", orc.PHIS)
def test_jagged_equals_independent_samples(phi):
    inp = problem(1, (5, 0, 9, 3), (4, 2, 7, 1))
    o, lse = orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, phi, kv_offsets=inp.kv_offsets)
    dq, dk, dv = orc.gdpa_backward(inp.q, inp.offsets, inp.k, inp.v, inp.do, phi, kv_offsets=inp.kv_offsets)
    off, ko = inp.offsets.numpy(), inp.kv_offsets.numpy()
    for b in range(4):
        r, c = slice(off[b], off[b + 1]), slice(ko[b], ko[b + 1])
        one = np.array([0, off[b + 1] - off[b]])
        kb, vb = inp.k[c].unsqueeze(0), inp.v[c].unsqueeze(0)
        ob, lb = orc.gdpa_forward(inp.q[r], one, kb, vb, phi)
        gq, gk, gv = orc.gdpa_backward(inp.q[r], one, kb, vb, inp.do[r], phi)
        assert np.array_equal(o[r], ob)
        assert np.array_equal(dq[r], gq) and np.array_equal(dk[c], gk[0]) and np.array_equal(dv[c], gv[0])
        if lse is not None:
            assert np.array_equal(lse[r], lb)


@pytest.mark.parametrize("phi", ["silu", "relu", "gelu", "identity"])
def test_elementwise_equals_zero_padded_dense(phi):
    inp = problem(2, (6, 4, 11), (3, 9, 5))
    kd, vd = padded(inp, 9)
    o, _ = orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, phi, kv_offsets=inp.kv_offsets)
    od, _ = orc.gdpa_forward(inp.q, inp.offsets, kd, vd, phi)
    assert rel(o, od) <= 1e-13
    dq, dk, dv = orc.gdpa_backward(inp.q, inp.offsets, inp.k, inp.v, inp.do, phi, kv_offsets=inp.kv_offsets)
    gq, gk, gv = orc.gdpa_backward(inp.q, inp.offsets, kd, vd, inp.do, phi)
    assert rel(dq, gq) <= 1e-13
    ko = inp.kv_offsets.numpy()
    for b in range(3):
        c = ko[b + 1] - ko[b]
        assert rel(dv[ko[b]:ko[b + 1]], gv[b, :c]) <= 1e-13
        assert rel(dk[ko[b]:ko[b + 1]], gk[b, :c]) <= 1e-13


def test_softmax_is_not_zero_padding():
    inp = problem(3, (6, 4), (3, 9))
    kd, vd = padded(inp, 9)
    o, _ = orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, "softmax", kv_offsets=inp.kv_offsets)
    od, _ = orc.gdpa_forward(inp.q, inp.offsets, kd, vd, "softmax")
    assert rel(o[:6], od[:6]) > 1e-3    # sample 0 would also weigh the 6 zero rows
    assert rel(o[6:], od[6:]) <= 1e-13  # sample 1 fills all 9 rows


def test_softmax_matches_torch_sdpa_per_sample():
    inp = problem(4, (7, 1, 12), (5, 13, 2), H=3, d=16)
    o, lse = orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, "softmax", kv_offsets=inp.kv_offsets)
    off, ko = inp.offsets.numpy(), inp.kv_offsets.numpy()
    for b in range(3):
        x = inp.q[off[b]:off[b + 1]].double().transpose(0, 1)
        kb = inp.k[ko[b]:ko[b + 1]].double().transpose(0, 1)
        vb = inp.v[ko[b]:ko[b + 1]].double().transpose(0, 1)
        ref = F.scaled_dot_product_attention(x, kb, vb, scale=1 / math.sqrt(16)).transpose(0, 1)
        assert rel(o[off[b]:off[b + 1]], ref.numpy()) <= 1e-13


def test_rejects_empty_context_and_bad_offsets():
    inp = problem(5, (3, 2), (2, 2))
    bad = torch.tensor([0, 2, 2, 4], dtype=torch.int32)
    q3 = torch.zeros((6, 2, 8))
    with pytest.raises(ValueError):
        orc.gdpa_forward(q3, np.array([0, 3, 4, 6]), inp.k, inp.v, "softmax", kv_offsets=bad)
    with pytest.raises(ValueError):
        orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, "softmax", kv_offsets=torch.tensor([0, 2, 5]))
