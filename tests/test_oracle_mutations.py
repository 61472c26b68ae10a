"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch them.

Each mutant replaces one piece of the oracle for the duration of a test; the
pin that should notice it is then run and must fail.  This shows the pins are
sharp enough to detect a dropped term, a wrong sign, a missing scale or a
transposed operand.
"""
import numpy as np
import pytest

from oracle import gdpa_oracle as orc
from oracle.brute import brute_forward
from tests.test_oracle_pins import fd_check, rand_problem, rel_err, torch_grads


def _wrong_silu_grad(s):
    g = orc.sigmoid(s)
    return g * (1.0 + s * g)                     # sign slip inside the bracket


def _wrong_softmax(s):
    m = s.max(axis=0, keepdims=True)            # normalised over the wrong axis
    e = np.exp(s - m)
    l = e.sum(axis=0, keepdims=True)
    return e / l, np.log(np.exp(s).sum(axis=-1))


def _backward_factory(kind):
    def bwd(x, kb, vb, do, phi, scale, sbias=None, with_bias_grads=False):
        s = scale * (x @ kb.T)
        if sbias is not None:
            s = s + sbias[None, :]
        dp = do @ vb.T
        if phi == "softmax":
            p, _ = orc.row_softmax(s)
            o = p @ vb
            dvec = (do * o).sum(axis=-1, keepdims=True)
            ds = p * dp if kind == "drop_D" else p * (dp - dvec)
        else:
            p = orc.silu(s)
            ds = dp * orc.silu_grad(s)
        dv = (do.T @ p).T if kind != "transpose_dv" else (p.T @ do)[::-1]
        dx = scale * (ds @ kb)
        dk = (ds.T @ x) if kind == "no_scale_dk" else scale * (ds.T @ x)
        if with_bias_grads:
            return dx, dk, dv, ds.sum(axis=0), do.sum(axis=0)
        return dx, dk, dv
    return bwd


def _torch_pin(phi):
    off, q, k, v = rand_problem(8, (5, 0, 7, 1), H=2, d=4, n=3, sharp=True)
    g = np.random.default_rng(9).standard_normal(q.shape)
    dq, dk, dv = orc.gdpa_backward(q, off, k, v, g, phi, None)
    tq, tk, tv = torch_grads(q, off, k, v, g, phi, orc.default_scale(phi, 4))
    return max(rel_err(dq, tq), rel_err(dk, tk), rel_err(dv, tv))


def test_mutant_silu_grad_is_caught(monkeypatch):
    monkeypatch.setattr(orc, "silu_grad", _wrong_silu_grad)
    assert fd_check("silu", None) > 1e-3
    assert _torch_pin("silu") > 1e-3


def test_mutant_gelu_grad_is_caught(monkeypatch):
    monkeypatch.setattr(orc, "gelu_grad", lambda s: orc.normal_cdf(s))  # density term dropped
    assert fd_check("gelu", None) > 1e-3
    assert _torch_pin("gelu") > 1e-3


def test_mutant_relu_is_caught(monkeypatch):
    monkeypatch.setattr(orc, "relu", lambda s: np.abs(s))  # |s| instead of max(s, 0)
    off, q, k, v = rand_problem(4, (4, 2), H=1, d=4, n=3, sharp=True)
    o, _ = orc.gdpa_forward(q, off, k, v, "relu", 0.5)
    ob, _ = brute_forward(q.tolist(), off.tolist(), k.tolist(), v.tolist(), "relu", 0.5)
    assert rel_err(o, np.array(ob)) > 1e-3


def test_mutant_softmax_axis_is_caught(monkeypatch):
    off, q, k, v = rand_problem(3, (4, 2), H=1, d=4, n=3, sharp=True)
    monkeypatch.setattr(orc, "row_softmax", _wrong_softmax)
    o, _ = orc.gdpa_forward(q, off, k, v, "softmax", 0.5)
    ob, _ = brute_forward(q.tolist(), off.tolist(), k.tolist(), v.tolist(), "softmax", 0.5)
    assert rel_err(o, np.array(ob)) > 1e-3


@pytest.mark.parametrize("kind,phi", [("drop_D", "softmax"), ("no_scale_dk", "softmax"),
                                      ("no_scale_dk", "silu"), ("transpose_dv", "silu")])
def test_mutant_backward_is_caught(monkeypatch, kind, phi):
    monkeypatch.setattr(orc, "gdpa_backward_bh", _backward_factory(kind))
    scale = 0.6 if kind == "no_scale_dk" else None
    assert fd_check(phi, scale) > 1e-3


def test_unmutated_backward_factory_passes(monkeypatch):
    # The mutant scaffolding itself is faithful when no mutation is selected.
    monkeypatch.setattr(orc, "gdpa_backward_bh", _backward_factory("none"))
    assert fd_check("softmax", 0.6) <= 1e-6 and fd_check("silu", None) <= 1e-6
