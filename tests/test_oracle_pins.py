"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each check ties the oracle to something independent: a scalar brute force, a
library routine the definition reduces to (torch's scaled-dot-product attention,
torch's SiLU / ReLU / GELU and linear layers, torch autograd), a closed form, an algebraic
invariant or central finite differences.  GDPA definition: Kunlun paper summary,
section 2.2 (GDPA bullet) and Telegram review, layer steps 1-2.
"""
import math
import zlib

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import gdpa_oracle as orc
from oracle.brute import brute_forward

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def rand_problem(seed, lengths, H, d, n, sharp=False):
    rng = np.random.default_rng(seed)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T, B = int(off[-1]), len(lengths)
    sc = 1.0 if sharp else 1.0 / math.sqrt(d)
    q = rng.standard_normal((T, H, d)) * sc
    k = rng.standard_normal((B, n, H, d)) * sc
    v = rng.standard_normal((B, n, H, d)) / math.sqrt(d)
    return off, q, k, v


def rel_err(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    den = max(np.abs(b).max(), 1e-300) if b.size else 1.0
    return float(np.abs(a - b).max() / den) if b.size else 0.0


# ---------------------------------------------------------------------------
# Brute force on tiny inputs
# ---------------------------------------------------------------------------

ALL_PHIS = ["softmax", "silu", "relu", "gelu", "identity"]
TORCH_ACT = {"silu": F.silu, "relu": F.relu, "gelu": F.gelu, "identity": lambda x: x}


@pytest.mark.parametrize("phi", ALL_PHIS)
@pytest.mark.parametrize("scale", [0.5, 1.0])
@pytest.mark.parametrize("lengths", [(3,), (2, 0, 5), (0, 1, 4), (5, 5, 1)])
def test_brute_force_tiny(phi, scale, lengths):
    off, q, k, v = rand_problem(zlib.crc32(repr((phi, scale, lengths)).encode()) % 1000, lengths, H=2, d=4, n=3, sharp=True)
    o, lse = orc.gdpa_forward(q, off, k, v, phi, scale)
    ob, lseb = brute_forward(q.tolist(), off.tolist(), k.tolist(), v.tolist(), phi, scale)
    if o.size:
        assert rel_err(o, np.array(ob)) <= 1e-13
    if phi == "softmax" and o.size:
        assert np.abs(lse - np.array(lseb)).max() <= 1e-13


# ---------------------------------------------------------------------------
# SiLU form: the per-sample two-layer FFN silu(x K^T) V
# ---------------------------------------------------------------------------

def ffn_torch(x, kb, vb, scale=1.0, act=F.silu):
    """Two bias-free linear layers with an activation between, in torch fp64."""
    x, kb, vb = (torch.from_numpy(a) for a in (x, kb, vb))
    hid = act(F.linear(x, kb) * scale)
    return F.linear(hid, vb.T.contiguous()).numpy()


@pytest.mark.parametrize("phi", ["relu", "gelu"])
def test_elementwise_equals_two_layer_ffn(phi):
    # torch's relu and (exact, erf-form) gelu between two bias-free linear layers.
    off, q, k, v = rand_problem(31, (7, 0, 13, 4), H=3, d=8, n=6, sharp=True)
    for scale in (1.0, 0.6):
        o, lse = orc.gdpa_forward(q, off, k, v, phi, scale)
        assert lse is None
        for b in range(4):
            for h in range(3):
                r = slice(off[b], off[b + 1])
                ref = ffn_torch(q[r, h, :], k[b, :, h, :], v[b, :, h, :], scale, TORCH_ACT[phi])
                assert rel_err(o[r, h, :], ref) <= 1e-13


def test_identity_is_bilinear():
    # phi = identity: O = scale (X K^T) V = scale X (K^T V) (associativity), linear in X.
    off, q, k, v = rand_problem(32, (6, 0, 3), H=2, d=5, n=4, sharp=True)
    o, _ = orc.gdpa_forward(q, off, k, v, "identity", 0.7)
    for b in range(3):
        for h in range(2):
            r = slice(off[b], off[b + 1])
            ref = 0.7 * (q[r, h, :] @ (k[b, :, h, :].T @ v[b, :, h, :]))
            if ref.size:
                assert np.abs(o[r, h, :] - ref).max() <= 1e-13 * max(1.0, np.abs(ref).max())
    o2, _ = orc.gdpa_forward(2.5 * q, off, k, v, "identity", 0.7)
    assert rel_err(o2, 2.5 * o) <= 1e-14


def test_relu_gelu_special_cases():
    rng = np.random.default_rng(33)
    d = 5
    x = rng.standard_normal((6, d))
    eye = np.eye(d)
    vb = rng.standard_normal((d, 3))
    # K = I: O = phi(X) V with torch's own activations.
    for phi in ("relu", "gelu"):
        o, _ = orc.gdpa_forward_bh(x, eye, vb, phi, 1.0)
        ref = TORCH_ACT[phi](torch.from_numpy(x)).numpy() @ vb
        assert rel_err(o, ref) <= 1e-14
    # GELU: Phi(s) + Phi(-s) = 1, so gelu(s) - gelu(-s) = s.
    s = np.linspace(-6.0, 6.0, 241)
    assert np.abs(orc.gelu(s) - orc.gelu(-s) - s).max() <= 1e-14
    assert orc.gelu(np.array([0.0]))[0] == 0.0
    # ReLU is positively homogeneous: a scale c > 0 scales the output.
    kb = rng.standard_normal((4, d))
    vb4 = rng.standard_normal((4, d))
    o1, _ = orc.gdpa_forward_bh(x, kb, vb4, "relu", 0.5)
    o2, _ = orc.gdpa_forward_bh(x, kb, vb4, "relu", 1.5)
    assert rel_err(o2, 3.0 * o1) <= 1e-14


def test_silu_equals_two_layer_ffn():
    off, q, k, v = rand_problem(1, (7, 0, 13, 4), H=3, d=8, n=6, sharp=True)
    o, lse = orc.gdpa_forward(q, off, k, v, "silu")
    assert lse is None
    for b in range(4):
        for h in range(3):
            r = slice(off[b], off[b + 1])
            ref = ffn_torch(q[r, h], k[b, :, h], v[b, :, h])
            assert rel_err(o[r, h], ref) <= 1e-13


def test_silu_special_cases():
    d = 5
    rng = np.random.default_rng(2)
    x = rng.standard_normal((9, d)) * 2
    vb = rng.standard_normal((d, d))
    eye = np.eye(d)
    # K = 0: silu(0) = 0 so the output vanishes.
    o, _ = orc.gdpa_forward_bh(x, np.zeros((4, d)), rng.standard_normal((4, d)), "silu", 1.0)
    assert np.all(o == 0.0)
    # K = I: O = silu(X) V, with torch's own SiLU.
    o, _ = orc.gdpa_forward_bh(x, eye, vb, "silu", 1.0)
    ref = F.silu(torch.from_numpy(x)).numpy() @ vb
    assert rel_err(o, ref) <= 1e-14
    # V = I: O = silu(X K^T).
    kb = rng.standard_normal((d, d))
    o, _ = orc.gdpa_forward_bh(x, kb, eye, "silu", 1.0)
    assert rel_err(o, F.silu(torch.from_numpy(x @ kb.T)).numpy()) <= 1e-14
    # Linearity in V.
    o1, _ = orc.gdpa_forward_bh(x, kb, vb, "silu", 0.7)
    o2, _ = orc.gdpa_forward_bh(x, kb, 3.0 * vb, "silu", 0.7)
    assert rel_err(o2, 3.0 * o1) <= 1e-14


def test_silu_extreme_scores_are_finite():
    x = np.array([[1.0]])
    kb = np.array([[800.0], [-800.0], [0.0]])
    vb = np.array([[1.0], [1.0], [1.0]])
    o, _ = orc.gdpa_forward_bh(x, kb, vb, "silu", 1.0)
    # silu(800) = 800, silu(-800) = -800 * e^-800 ~ 0, silu(0) = 0
    assert o[0, 0] == pytest.approx(800.0, rel=1e-15)


# ---------------------------------------------------------------------------
# Softmax form: naive attention
# ---------------------------------------------------------------------------

def test_softmax_equals_torch_sdpa():
    off, q, k, v = rand_problem(3, (6, 1, 0, 11), H=2, d=8, n=5, sharp=True)
    for scale in (None, 0.3):
        o, lse = orc.gdpa_forward(q, off, k, v, "softmax", scale)
        sc = 1 / math.sqrt(8) if scale is None else scale
        for b in range(4):
            r = slice(off[b], off[b + 1])
            if off[b] == off[b + 1]:
                continue
            for h in range(2):
                qt = torch.from_numpy(q[r, h])[None]
                kt = torch.from_numpy(k[b, :, h])[None]
                vt = torch.from_numpy(v[b, :, h])[None]
                ref = F.scaled_dot_product_attention(qt, kt, vt, scale=sc)[0].numpy()
                assert rel_err(o[r, h], ref) <= 1e-13
                s = sc * (q[r, h] @ k[b, :, h].T)
                lse_ref = torch.logsumexp(torch.from_numpy(s), dim=-1).numpy()
                assert np.abs(lse[r, h] - lse_ref).max() <= 1e-13


def test_softmax_rows_sum_to_one_and_lse():
    off, q, k, v = rand_problem(4, (9, 3), H=2, d=4, n=7, sharp=True)
    ones = np.ones_like(v)
    o, lse = orc.gdpa_forward(q, off, k, ones, "softmax")
    assert np.abs(o - 1.0).max() <= 1e-14
    sc = 1 / 2.0
    for b in range(2):
        r = slice(off[b], off[b + 1])
        for h in range(2):
            s = sc * q[r, h] @ k[b, :, h].T
            assert np.abs(np.exp(s - lse[r, h][:, None]).sum(-1) - 1.0).max() <= 1e-14


def test_softmax_closed_forms():
    rng = np.random.default_rng(5)
    # n = 1: every row is that one V row.
    x = rng.standard_normal((4, 3))
    kb, vb = rng.standard_normal((1, 3)), rng.standard_normal((1, 3))
    o, lse = orc.gdpa_forward_bh(x, kb, vb, "softmax", 0.9)
    assert np.all(o == vb[0])
    assert np.allclose(lse, 0.9 * (x @ kb[0]), rtol=0, atol=1e-15)
    # n = 2, d = 1: O = v1 sigmoid(s1 - s2) + v2 sigmoid(s2 - s1).
    x = np.array([[0.3], [-1.7], [2.2]])
    kb = np.array([[1.1], [-0.4]])
    vb = np.array([[2.0], [-3.0]])
    o, _ = orc.gdpa_forward_bh(x, kb, vb, "softmax", 1.0)
    for i in range(3):
        s1, s2 = x[i, 0] * 1.1, x[i, 0] * -0.4
        lg = lambda z: 1 / (1 + math.exp(-z))  # noqa: E731
        assert o[i, 0] == pytest.approx(2.0 * lg(s1 - s2) - 3.0 * lg(s2 - s1), abs=1e-15)
    # K = 0: uniform weights, O = mean of V rows.
    vb = rng.standard_normal((6, 3))
    o, lse = orc.gdpa_forward_bh(rng.standard_normal((5, 3)), np.zeros((6, 3)), vb, "softmax", 1.0)
    assert np.abs(o - vb.mean(0)).max() <= 1e-15
    assert np.abs(lse - math.log(6)).max() <= 1e-15


def test_softmax_invariances():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((8, 4))
    kb, vb = rng.standard_normal((5, 4)), rng.standard_normal((5, 4))
    o, _ = orc.gdpa_forward_bh(x, kb, vb, "softmax", 0.8)
    u, w = rng.standard_normal(4), rng.standard_normal(4)
    # Adding the same vector to every key row shifts each score row by a constant.
    o2, _ = orc.gdpa_forward_bh(x, kb + u, vb, "softmax", 0.8)
    assert rel_err(o2, o) <= 1e-13
    # Adding w to every value row adds w to every output row.
    o3, _ = orc.gdpa_forward_bh(x, kb, vb + w, "softmax", 0.8)
    assert rel_err(o3, o + w) <= 1e-13
    # Permuting context rows jointly in K and V changes nothing.
    perm = rng.permutation(5)
    o4, _ = orc.gdpa_forward_bh(x, kb[perm], vb[perm], "softmax", 0.8)
    assert rel_err(o4, o) <= 1e-14


def test_softmax_extreme_scores_are_finite():
    x = np.array([[1.0], [-1.0]])
    kb = np.array([[900.0], [899.0], [-900.0]])
    vb = np.array([[1.0], [0.0], [5.0]])
    o, lse = orc.gdpa_forward_bh(x, kb, vb, "softmax", 1.0)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert o[0, 0] == pytest.approx(1 / (1 + math.exp(-1)), rel=1e-14)
    assert o[1, 0] == pytest.approx(5.0, rel=1e-14)


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------

def fd_check(phi, scale, seed=7, h=1e-6):
    """Worst |fd - analytic| / max(1, |analytic|) over every element of Q, K, V."""
    off, q, k, v = rand_problem(seed, (2, 0, 3), H=2, d=4, n=3, sharp=True)
    rng = np.random.default_rng(seed + 100)
    g = rng.standard_normal(q.shape)
    dq, dk, dv = orc.gdpa_backward(q, off, k, v, g, phi, scale)

    def loss(q_, k_, v_):
        o, _ = orc.gdpa_forward(q_, off, k_, v_, phi, scale)
        return float((o * g).sum())

    worst = 0.0
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        flat = arr.reshape(-1)
        gflat = grad.reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + h
            lp = loss(q, k, v)
            flat[i] = old - h
            lm = loss(q, k, v)
            flat[i] = old
            fd = (lp - lm) / (2 * h)
            worst = max(worst, abs(fd - gflat[i]) / max(1.0, abs(gflat[i])))
    return worst


@pytest.mark.parametrize("phi", ALL_PHIS)
@pytest.mark.parametrize("scale", [None, 0.6])
def test_backward_finite_differences(phi, scale):
    assert fd_check(phi, scale) <= 1e-6


def torch_grads(q, off, k, v, g, phi, scale):
    """Autograd of the jagged op built from torch library ops (SDPA / matmul + activation)."""
    qt = torch.from_numpy(q.copy()).requires_grad_()
    kt = torch.from_numpy(k.copy()).requires_grad_()
    vt = torch.from_numpy(v.copy()).requires_grad_()
    outs = []
    B = k.shape[0]
    for b in range(B):
        xb = qt[off[b]:off[b + 1]].transpose(0, 1)          # [H, L, d]
        kb = kt[b].transpose(0, 1)
        vb = vt[b].transpose(0, 1)
        if phi == "softmax":
            ob = F.scaled_dot_product_attention(xb, kb, vb, scale=scale)
        else:
            ob = TORCH_ACT[phi](torch.matmul(xb, kb.transpose(1, 2)) * scale) @ vb
        outs.append(ob.transpose(0, 1))
    o = torch.cat(outs, 0)
    (o * torch.from_numpy(g)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("phi", ALL_PHIS)
def test_backward_matches_torch_autograd(phi):
    lengths = (5, 0, 17, 1, 9)
    off, q, k, v = rand_problem(8, lengths, H=3, d=8, n=6, sharp=True)
    g = np.random.default_rng(9).standard_normal(q.shape)
    scale = orc.default_scale(phi, 8)
    dq, dk, dv = orc.gdpa_backward(q, off, k, v, g, phi, None)
    tq, tk, tv = torch_grads(q, off, k, v, g, phi, scale)
    assert rel_err(dq, tq) <= 1e-12
    assert rel_err(dk, tk) <= 1e-12
    assert rel_err(dv, tv) <= 1e-12


def test_softmax_backward_invariants():
    off, q, k, v = rand_problem(10, (6, 3, 0), H=2, d=4, n=5, sharp=True)
    g = np.random.default_rng(11).standard_normal(q.shape)
    dq, dk, dv = orc.gdpa_backward(q, off, k, v, g, "softmax")
    for b in range(3):
        # Softmax is invariant to a common shift of the key rows -> sum_j dK = 0.
        assert np.abs(dk[b].sum(0)).max() <= 1e-13
        # Rows of P sum to 1 -> sum_j dV[j] = sum_t dO[t].
        ref = g[off[b]:off[b + 1]].sum(0)
        assert np.abs(dv[b].sum(0) - ref).max() <= 1e-13
    # Empty sample: zero dK and dV.
    assert np.all(dk[2] == 0) and np.all(dv[2] == 0)
    # n = 1: P = 1 whatever the scores -> dQ = dK = 0 (up to the rounding of dP - D).
    off1, q1, k1, v1 = rand_problem(12, (4, 2), H=2, d=3, n=1)
    g1 = np.random.default_rng(13).standard_normal(q1.shape)
    dq1, dk1, dv1 = orc.gdpa_backward(q1, off1, k1, v1, g1, "softmax")
    assert np.abs(dq1).max() <= 1e-15 and np.abs(dk1).max() <= 1e-15


def test_silu_backward_linear_in_v_and_do():
    off, q, k, v = rand_problem(14, (5, 2), H=1, d=4, n=3, sharp=True)
    g = np.random.default_rng(15).standard_normal(q.shape)
    dq, dk, dv = orc.gdpa_backward(q, off, k, v, g, "silu")
    dq2, dk2, dv2 = orc.gdpa_backward(q, off, k, 2.0 * v, g, "silu")
    # dV does not depend on V; dQ and dK are linear in V.
    assert rel_err(dv2, dv) <= 1e-14
    assert rel_err(dq2, 2 * dq) <= 1e-14 and rel_err(dk2, 2 * dk) <= 1e-14


# ---------------------------------------------------------------------------
# Jagged-batch semantics
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("phi", ALL_PHIS)
def test_jagged_equals_independent_samples(phi):
    lengths = (4, 0, 9, 1)
    off, q, k, v = rand_problem(16, lengths, H=2, d=4, n=3, sharp=True)
    g = np.random.default_rng(17).standard_normal(q.shape)
    o, lse = orc.gdpa_forward(q, off, k, v, phi)
    dq, dk, dv = orc.gdpa_backward(q, off, k, v, g, phi)
    for b in range(4):
        r = slice(off[b], off[b + 1])
        ob, _ = orc.gdpa_forward(q[r], np.array([0, lengths[b]]), k[b:b + 1], v[b:b + 1], phi)
        assert np.array_equal(ob, o[r])
        gq, gk, gv = orc.gdpa_backward(q[r], np.array([0, lengths[b]]), k[b:b + 1], v[b:b + 1],
                                       g[r], phi)
        assert np.array_equal(gq, dq[r]) and np.array_equal(gk[0], dk[b]) and np.array_equal(gv[0], dv[b])
    # Permuting samples permutes the outputs.
    perm = [2, 0, 3, 1]
    qs = np.concatenate([q[off[b]:off[b + 1]] for b in perm])
    offp = np.concatenate([[0], np.cumsum([lengths[b] for b in perm])])
    op, _ = orc.gdpa_forward(qs, offp, k[perm], v[perm], phi)
    assert np.array_equal(op, np.concatenate([o[off[b]:off[b + 1]] for b in perm]))


# ---------------------------------------------------------------------------
# Stacked layers with generated K/V
# ---------------------------------------------------------------------------

def stacked_problem(seed=18, lengths=(3, 0, 5), H=2, d=4, n=3, C=5, layers=2):
    rng = np.random.default_rng(seed)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(off[-1])
    x0 = rng.standard_normal((T, H * d))
    ctx = rng.standard_normal((len(lengths), C))
    wk = [rng.standard_normal((n * H * d, C)) * 0.3 for _ in range(layers)]
    wv = [rng.standard_normal((n * H * d, C)) * 0.3 for _ in range(layers)]
    g = rng.standard_normal((T, H * d))
    return off, x0, ctx, wk, wv, g


@pytest.mark.parametrize("phi", ["silu", "softmax"])
def test_stacked_matches_torch_autograd(phi):
    off, x0, ctx, wk, wv, g = stacked_problem()
    H, n, d = 2, 3, 4
    xs = orc.stacked_forward(x0, off, ctx, wk, wv, H, n, phi)
    dx0, dwk, dwv = orc.stacked_backward(xs, off, ctx, wk, wv, g, H, n, phi)
    # torch fp64 autograd of the same graph, built from linear layers and SiLU (the FFN
    # form) or a row softmax at scale 1/sqrt(d) (attention).
    xt = torch.from_numpy(x0.copy()).requires_grad_()
    ct = torch.from_numpy(ctx)
    wkt = [torch.from_numpy(w.copy()).requires_grad_() for w in wk]
    wvt = [torch.from_numpy(w.copy()).requires_grad_() for w in wv]
    x = xt
    for l in range(2):
        kl = torch.nn.functional.linear(ct, wkt[l]).reshape(3, n, H, d)
        vl = torch.nn.functional.linear(ct, wvt[l]).reshape(3, n, H, d)
        rows = []
        for b in range(3):
            xb = x[off[b]:off[b + 1]].reshape(-1, H, d).transpose(0, 1)
            sc = xb @ kl[b].transpose(0, 1).transpose(1, 2)
            pm = F.silu(sc) if phi == "silu" else torch.softmax(sc / math.sqrt(d), dim=-1)
            ob = pm @ vl[b].transpose(0, 1)
            rows.append(ob.transpose(0, 1).reshape(-1, H * d))
        x = x + torch.cat(rows, 0)
        assert rel_err(xs[l + 1], x.detach().numpy()) <= 1e-13
    (x * torch.from_numpy(g)).sum().backward()
    assert rel_err(dx0, xt.grad.numpy()) <= 1e-12
    for l in range(2):
        assert rel_err(dwk[l], wkt[l].grad.numpy()) <= 1e-12
        assert rel_err(dwv[l], wvt[l].grad.numpy()) <= 1e-12


def test_stacked_weight_gradient_finite_differences():
    off, x0, ctx, wk, wv, g = stacked_problem(seed=19, lengths=(2, 3), C=3, layers=2)
    H, n = 2, 3
    xs = orc.stacked_forward(x0, off, ctx, wk, wv, H, n, "silu")
    _, dwk, dwv = orc.stacked_backward(xs, off, ctx, wk, wv, g, H, n, "silu")

    def loss():
        return float((orc.stacked_forward(x0, off, ctx, wk, wv, H, n, "silu")[-1] * g).sum())

    h = 1e-6
    rng = np.random.default_rng(20)
    for ws, gs in ((wk, dwk), (wv, dwv)):
        for l in range(2):
            for i in rng.choice(ws[l].size, 12, replace=False):
                flat = ws[l].reshape(-1)
                old = flat[i]
                flat[i] = old + h
                lp = loss()
                flat[i] = old - h
                lm = loss()
                flat[i] = old
                an = gs[l].reshape(-1)[i]
                assert abs((lp - lm) / (2 * h) - an) <= 1e-6 * max(1.0, abs(an))
