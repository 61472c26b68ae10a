"""Pins of the sliding-window self-attention oracle against independent facts:
a scalar brute force, torch's scaled-dot-product attention with a causal flag or
an explicit band mask (forward and autograd), closed forms (window 1), causality
and locality invariants, and central finite differences.  Definition: Kunlun
paper summary, section 2.2 (Sliding Window Attention bullet); Telegram review,
layer step 5 and the event-level personalisation list (w, the window size)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import swa_oracle as swa
from oracle.brute import brute_swa_forward

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def problem(seed, lengths, H, d, sharp=True):
    rng = np.random.default_rng(seed)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(off[-1])
    sc = 1.0 if sharp else 1.0 / math.sqrt(d)
    q = rng.standard_normal((T, H, d)) * sc
    k = rng.standard_normal((T, H, d)) * sc
    v = rng.standard_normal((T, H, d))
    return off, q, k, v


def rel_err(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    if b.size == 0:
        return 0.0
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


def sdpa_ref(q, off, k, v, window, scale, grad_out=None):
    """torch SDPA per sample with a boolean band mask (True = attend), fp64; with
    grad_out also the autograd gradients."""
    qt, kt, vt = (torch.from_numpy(a.copy()).requires_grad_() for a in (q, k, v))
    outs = []
    for b in range(len(off) - 1):
        r = slice(int(off[b]), int(off[b + 1]))
        L = r.stop - r.start
        if L == 0:
            continue
        mask = torch.from_numpy(swa.band_mask(L, window))
        ob = F.scaled_dot_product_attention(qt[r].transpose(0, 1), kt[r].transpose(0, 1),
                                            vt[r].transpose(0, 1), attn_mask=mask, scale=scale)
        outs.append(ob.transpose(0, 1))
    o = torch.cat(outs, 0)
    if grad_out is None:
        return o.detach().numpy()
    (o * torch.from_numpy(grad_out)).sum().backward()
    return o.detach().numpy(), qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("window", [1, 2, 3, 7])
@pytest.mark.parametrize("lengths", [(5,), (3, 0, 6), (1, 4)])
def test_brute_force_tiny(window, lengths):
    off, q, k, v = problem(window * 10 + len(lengths), lengths, H=2, d=3)
    o, lse = swa.swa_forward(q, off, k, v, window, 0.7)
    ob, lb = brute_swa_forward(q.tolist(), off.tolist(), k.tolist(), v.tolist(), window, 0.7)
    if o.size:
        assert rel_err(o, np.array(ob)) <= 1e-13
        assert np.abs(lse - np.array(lb)).max() <= 1e-13


@pytest.mark.parametrize("window", [1, 5, 16, 1000])
def test_forward_equals_torch_sdpa_with_band_mask(window):
    off, q, k, v = problem(1, (9, 0, 23, 1, 40), H=3, d=8)
    o, _ = swa.swa_forward(q, off, k, v, window)
    assert rel_err(o, sdpa_ref(q, off, k, v, window, 1 / math.sqrt(8))) <= 1e-13


def test_long_window_is_causal_attention():
    # w >= L: plain causal attention (torch's is_causal flag, no explicit mask).
    off, q, k, v = problem(2, (17, 5), H=2, d=4)
    o, _ = swa.swa_forward(q, off, k, v, 64, 0.5)
    for b in range(2):
        r = slice(off[b], off[b + 1])
        ref = F.scaled_dot_product_attention(*(torch.from_numpy(a[r]).transpose(0, 1) for a in (q, k, v)),
                                             is_causal=True, scale=0.5).transpose(0, 1).numpy()
        assert rel_err(o[r], ref) <= 1e-13


def test_window_one_closed_form():
    # Each token sees only itself: O = V and LSE = its own score.
    off, q, k, v = problem(3, (6, 2), H=2, d=5)
    o, lse = swa.swa_forward(q, off, k, v, 1, 0.3)
    assert rel_err(o, v) <= 1e-15
    assert np.abs(lse - 0.3 * (q * k).sum(-1)).max() <= 1e-13


def test_causality_and_locality():
    off, q, k, v = problem(4, (30,), H=1, d=4)
    w = 6
    o, _ = swa.swa_forward(q, off, k, v, w)
    # Appending later tokens changes nothing before them.
    o_short, _ = swa.swa_forward(q[:20], np.array([0, 20]), k[:20], v[:20], w)
    assert rel_err(o_short, o[:20]) <= 1e-14   # (different matrix shapes: rounding only)
    # Tokens more than w - 1 back do not matter: perturb token 5, rows >= 5 + w are unchanged.
    k2, v2 = k.copy(), v.copy()
    k2[5] += 3.0
    v2[5] -= 2.0
    o2, _ = swa.swa_forward(q, off, k2, v2, w)
    assert rel_err(o2[5 + w:], o[5 + w:]) <= 1e-14
    assert np.abs(o2[5:5 + w] - o[5:5 + w]).max() > 1e-3


def test_rows_of_p_sum_to_one():
    # V = 1 gives O = 1 for every token.
    off, q, k, v = problem(5, (11, 3), H=2, d=4)
    o, _ = swa.swa_forward(q, off, k, np.ones_like(v), 4)
    assert np.abs(o - 1.0).max() <= 1e-14


@pytest.mark.parametrize("window", [1, 3, 100])
def test_backward_matches_torch_autograd(window):
    off, q, k, v = problem(6, (7, 0, 12, 2), H=2, d=4)
    g = np.random.default_rng(7).standard_normal(q.shape)
    dq, dk, dv = swa.swa_backward(q, off, k, v, g, window, 0.6)
    _, tq, tk, tv = sdpa_ref(q, off, k, v, window, 0.6, g)
    assert rel_err(dv, tv) <= 1e-12
    if window == 1:
        # P = I: dS = dP - rowsum(dO O) vanishes on the diagonal, so dQ = dK = 0, dV = dO.
        assert np.abs(dq).max() <= 1e-13 and np.abs(dk).max() <= 1e-13
        assert np.abs(tq).max() <= 1e-13 and rel_err(dv, g) <= 1e-15
    else:
        assert rel_err(dq, tq) <= 1e-12 and rel_err(dk, tk) <= 1e-12


def test_backward_finite_differences():
    off, q, k, v = problem(8, (4, 0, 5), H=1, d=3)
    g = np.random.default_rng(9).standard_normal(q.shape)
    w, h = 3, 1e-6
    dq, dk, dv = swa.swa_backward(q, off, k, v, g, w, 0.8)

    def loss():
        return float((swa.swa_forward(q, off, k, v, w, 0.8)[0] * g).sum())

    worst = 0.0
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        flat, gflat = arr.reshape(-1), grad.reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + h
            lp = loss()
            flat[i] = old - h
            lm = loss()
            flat[i] = old
            worst = max(worst, abs((lp - lm) / (2 * h) - gflat[i]) / max(1.0, abs(gflat[i])))
    assert worst <= 1e-6


def test_jagged_equals_independent_samples():
    lengths = (8, 0, 13)
    off, q, k, v = problem(10, lengths, H=2, d=4)
    g = np.random.default_rng(11).standard_normal(q.shape)
    o, lse = swa.swa_forward(q, off, k, v, 5)
    dq, dk, dv = swa.swa_backward(q, off, k, v, g, 5)
    for b in range(3):
        r = slice(off[b], off[b + 1])
        sub = np.array([0, lengths[b]])
        ob, lb = swa.swa_forward(q[r], sub, k[r], v[r], 5)
        assert np.array_equal(ob, o[r]) and np.array_equal(lb, lse[r])
        gq, gk, gv = swa.swa_backward(q[r], sub, k[r], v[r], g[r], 5)
        assert np.array_equal(gq, dq[r]) and np.array_equal(gk, dk[r]) and np.array_equal(gv, dv[r])


def test_mutant_window_off_by_one_is_caught(monkeypatch):
    # A window that also admits token i - w (one too many) disagrees with the brute force.
    off, q, k, v = problem(12, (9,), H=1, d=3)
    monkeypatch.setattr(swa, "band_mask", lambda L, w: (np.arange(L)[None, :] <= np.arange(L)[:, None])
                        & (np.arange(L)[None, :] >= np.arange(L)[:, None] - w))
    o, _ = swa.swa_forward(q, off, k, v, 3, 0.7)
    ob, _ = brute_swa_forward(q.tolist(), off.tolist(), k.tolist(), v.tolist(), 3, 0.7)
    assert rel_err(o, np.array(ob)) > 1e-3
