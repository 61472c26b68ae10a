"""Shape fuzzing (hypothesis) of the oracle and of the host-side ABI checks.

* The vectorised oracle forward equals the scalar brute force (oracle/brute.py,
  explicit index loops) on random jagged batches: lengths including 0, any
  H, d, n, every map, random scale.
* The oracle backward equals a central finite difference of the oracle forward
  along a random direction of (q, k, v), for every map.
* gdpa_check_offsets / gdpa_check_kv_offsets accept exactly the arrays that the
  header's contract describes.
"""
import ctypes

import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

from oracle import gdpa_oracle as go  # noqa: E402
from oracle.brute import brute_forward  # noqa: E402

PHIS = ["softmax", "silu", "relu", "gelu", "identity"]


@st.composite
def problems(draw, max_len=6):
    B = draw(st.integers(0, 4))
    lengths = draw(st.lists(st.integers(0, max_len), min_size=B, max_size=B))
    H = draw(st.integers(1, 3))
    d = draw(st.integers(1, 5))
    n = draw(st.integers(1, 5))
    phi = draw(st.sampled_from(PHIS))
    scale = draw(st.floats(0.05, 2.0))
    seed = draw(st.integers(0, 2**31 - 1))
    return lengths, H, d, n, phi, scale, seed


def make(lengths, H, d, n, seed):
    rng = np.random.default_rng(seed)
    B, T = len(lengths), int(sum(lengths))
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64) if B else np.zeros(1, np.int64)
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((B, n, H, d))
    v = rng.standard_normal((B, n, H, d))
    return offsets, q, k, v


@settings(max_examples=60, deadline=None)
@given(problems())
def test_oracle_forward_equals_brute_force(prob):
    lengths, H, d, n, phi, scale, seed = prob
    offsets, q, k, v = make(lengths, H, d, n, seed)
    if len(lengths) == 0:
        return  # nothing to compare: no samples, no tokens
    o, lse = go.gdpa_forward(q, offsets, k, v, phi, scale)
    ob, lb = brute_forward(q.tolist(), offsets.tolist(), k.tolist(), v.tolist(), phi, scale)
    ob = np.array(ob, dtype=np.float64).reshape(o.shape)
    assert np.allclose(o, ob, rtol=1e-11, atol=1e-11)
    if phi == "softmax":
        assert np.allclose(lse, np.array(lb, dtype=np.float64).reshape(lse.shape), rtol=1e-12, atol=1e-12)
    else:
        assert lse is None


@settings(max_examples=40, deadline=None)
@given(problems(max_len=5))
def test_oracle_backward_equals_directional_difference(prob):
    lengths, H, d, n, phi, scale, seed = prob
    offsets, q, k, v = make(lengths, H, d, n, seed)
    rng = np.random.default_rng(seed + 1)
    do = rng.standard_normal(q.shape)
    dirs = [rng.standard_normal(x.shape) for x in (q, k, v)]
    dq, dk, dv = go.gdpa_backward(q, offsets, k, v, do, phi, scale)
    # An empty sample's dK, dV are zeros (its sum has no terms).
    for b, L in enumerate(lengths):
        if L == 0:
            assert not dk[b].any() and not dv[b].any()

    def f(eps):
        o, _ = go.gdpa_forward(q + eps * dirs[0], offsets, k + eps * dirs[1], v + eps * dirs[2], phi, scale)
        return float((o * do).sum())

    eps = 1e-6
    fd = (f(eps) - f(-eps)) / (2 * eps)
    an = float((dq * dirs[0]).sum() + (dk * dirs[1]).sum() + (dv * dirs[2]).sum())
    # ReLU's kink at 0 is hit with probability 0 by continuous draws.
    assert abs(fd - an) <= 1e-5 * max(1.0, abs(an)), (fd, an)


def _lib():
    cca = pytest.importorskip("context_cross_attention_amd")
    try:
        return cca, cca.load()
    except ImportError as e:
        pytest.skip(str(e))


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(-3, 12), min_size=1, max_size=8), st.integers(-2, 60), st.integers(-1, 12))
def test_check_offsets_matches_the_contract(offs, total, max_seqlen):
    import torch
    cca, lib = _lib()
    a = np.array(offs, dtype=np.int32)
    d = np.diff(a)
    ok = (total >= 0 and max_seqlen >= 0 and a[0] == 0 and bool((d >= 0).all()) and a[-1] == total
          and bool((d <= max_seqlen).all()))
    t = torch.tensor(a, dtype=torch.int32)
    got = lib.gdpa_check_offsets(ctypes.c_void_p(t.data_ptr()), len(a) - 1, total, max_seqlen)
    assert (got == 0) == ok, (offs, total, max_seqlen, got)


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(-3, 12), min_size=1, max_size=8), st.integers(-1, 6))
def test_check_kv_offsets_matches_the_contract(offs, n_kv):
    import torch
    cca, lib = _lib()
    a = np.array(offs, dtype=np.int32)
    d = np.diff(a)
    ok = n_kv >= 1 and a[0] == 0 and bool((d >= 1).all()) and bool((d <= n_kv).all())
    t = torch.tensor(a, dtype=torch.int32)
    got = lib.gdpa_check_kv_offsets(ctypes.c_void_p(t.data_ptr()), len(a) - 1, n_kv)
    assert (got == 0) == ok, (offs, n_kv, got)
