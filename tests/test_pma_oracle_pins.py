"""Pins of the seed pooling attention oracle against independent facts: torch's
scaled-dot-product attention with the seeds as queries (forward and autograd), a
scalar brute force, closed forms (K = 0 gives the mean of V; one token gives its
V), permutation invariance over a sample's tokens, empty samples, and finite
differences.  Definition: Kunlun paper summary, sections 2.1 and 2.2 (Hierarchical
Seed Pooling bullet); Telegram review, layer step 3."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import pma_oracle as pma

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def problem(seed, lengths, m, H, d):
    rng = np.random.default_rng(seed)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(off[-1])
    seeds = rng.standard_normal((m, H, d))
    k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, d))
    return off, seeds, k, v


def rel_err(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)) if b.size else 0.0


def torch_ref(seeds, off, k, v, scale, g=None):
    st, kt, vt = (torch.from_numpy(a.copy()).requires_grad_() for a in (seeds, k, v))
    outs = []
    for b in range(len(off) - 1):
        r = slice(int(off[b]), int(off[b + 1]))
        if r.stop == r.start:
            outs.append(torch.zeros(seeds.shape, dtype=torch.float64))
            continue
        ob = F.scaled_dot_product_attention(st.transpose(0, 1), kt[r].transpose(0, 1), vt[r].transpose(0, 1),
                                            scale=scale)
        outs.append(ob.transpose(0, 1))
    o = torch.stack(outs, 0)
    if g is None:
        return o.detach().numpy()
    (o * torch.from_numpy(g)).sum().backward()
    return o.detach().numpy(), st.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def test_forward_equals_torch_sdpa():
    off, seeds, k, v = problem(1, (7, 0, 40, 1), m=5, H=3, d=8)
    o, lse = pma.pma_forward(seeds, off, k, v)
    assert rel_err(o, torch_ref(seeds, off, k, v, 1 / math.sqrt(8))) <= 1e-13
    # LSE definition on one row.
    s = (seeds[2, 1] @ k[7:47, 1].T) / math.sqrt(8)
    assert lse[2, 2, 1] == pytest.approx(math.log(np.exp(s).sum()), rel=1e-13)


def test_brute_force_tiny():
    off, seeds, k, v = problem(2, (3, 0, 4), m=2, H=1, d=3)
    o, _ = pma.pma_forward(seeds, off, k, v, 0.7)
    for b in range(3):
        for s in range(2):
            rows = range(off[b], off[b + 1])
            sc = [0.7 * sum(seeds[s, 0, e] * k[j, 0, e] for e in range(3)) for j in rows]
            if not sc:
                assert np.all(o[b, s] == 0)
                continue
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            z = sum(w)
            for e in range(3):
                ref = sum(wi / z * v[j, 0, e] for wi, j in zip(w, rows))
                assert o[b, s, 0, e] == pytest.approx(ref, rel=1e-13, abs=1e-14)


def test_closed_forms_and_invariances():
    off, seeds, k, v = problem(3, (6, 1, 9), m=4, H=2, d=5)
    # K = 0: every token weighs the same, O = mean of the sample's V.
    o, _ = pma.pma_forward(seeds, off, np.zeros_like(k), v)
    for b in range(3):
        r = slice(off[b], off[b + 1])
        assert rel_err(o[b], np.broadcast_to(v[r].mean(0), o[b].shape)) <= 1e-14
    # A one-token sample pools to that token's V.
    o, _ = pma.pma_forward(seeds, off, k, v)
    assert rel_err(o[1], np.broadcast_to(v[6], o[1].shape)) <= 1e-15
    # Permuting a sample's tokens leaves its pooled output unchanged.
    perm = np.arange(16)
    perm[7:16] = perm[7:16][::-1]
    o2, _ = pma.pma_forward(seeds, off, k[perm], v[perm])
    assert rel_err(o2, o) <= 1e-14


def test_backward_matches_torch_autograd():
    off, seeds, k, v = problem(4, (5, 0, 12, 2), m=3, H=2, d=4)
    g = np.random.default_rng(5).standard_normal((4, 3, 2, 4))
    ds, dk, dv = pma.pma_backward(seeds, off, k, v, g, 0.6)
    _, ts, tk, tv = torch_ref(seeds, off, k, v, 0.6, g)
    assert rel_err(ds, ts) <= 1e-12 and rel_err(dk, tk) <= 1e-12 and rel_err(dv, tv) <= 1e-12


def test_backward_finite_differences():
    off, seeds, k, v = problem(6, (3, 0, 4), m=2, H=1, d=3)
    g = np.random.default_rng(7).standard_normal((3, 2, 1, 3))
    ds, dk, dv = pma.pma_backward(seeds, off, k, v, g, 0.9)
    h = 1e-6
    worst = 0.0
    for arr, grad in ((seeds, ds), (k, dk), (v, dv)):
        flat, gflat = arr.reshape(-1), grad.reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + h
            lp = float((pma.pma_forward(seeds, off, k, v, 0.9)[0] * g).sum())
            flat[i] = old - h
            lm = float((pma.pma_forward(seeds, off, k, v, 0.9)[0] * g).sum())
            flat[i] = old
            worst = max(worst, abs((lp - lm) / (2 * h) - gflat[i]) / max(1.0, abs(gflat[i])))
    assert worst <= 1e-6


def test_mutant_softmax_over_seeds_is_caught(monkeypatch):
    # Normalising over the seeds instead of the tokens disagrees with torch.
    off, seeds, k, v = problem(8, (6, 3), m=4, H=1, d=3)

    def wrong(s):
        e = np.exp(s - s.max(axis=0, keepdims=True))
        return e / e.sum(axis=0, keepdims=True), np.zeros(s.shape[0])

    monkeypatch.setattr(pma, "row_softmax", wrong)
    o, _ = pma.pma_forward(seeds, off, k, v)
    assert rel_err(o, torch_ref(seeds, off, k, v, 1 / math.sqrt(3))) > 1e-3
