"""The Python binding rejects caller-supplied tensors of the wrong shape, dtype or
layout before any library call (CPU tensors: every case holds one bad tensor, so
nothing reaches the device)."""
import pytest
import torch

import context_cross_attention_amd as cca

T, B, H, d, n = 12, 2, 2, 32, 4
bf = torch.bfloat16


def base():
    q = torch.zeros((T, H, d), dtype=bf)
    off = torch.tensor([0, 5, T], dtype=torch.int32)
    k = torch.zeros((B, n, H, d), dtype=bf)
    v = torch.zeros((B, n, H, d), dtype=bf)
    return q, off, k, v


def jagged():
    q, off, _, _ = base()
    kv_off = torch.tensor([0, 3, 7], dtype=torch.int32)
    k = torch.zeros((7, H, d), dtype=bf)
    v = torch.zeros((7, H, d), dtype=bf)
    return q, off, kv_off, k, v


def strided_q():
    return torch.zeros((H, T, d), dtype=bf).transpose(0, 1)   # [T, H, d], not contiguous


BAD_LSE = [(torch.zeros((T, H + 1)), ValueError), (torch.zeros((T, H), dtype=torch.float64), TypeError),
           (torch.zeros((H, T)).t(), ValueError)]


@pytest.mark.parametrize("lse,exc", BAD_LSE)
def test_fwd_rejects_bad_lse(lse, exc):
    q, off, k, v = base()
    with pytest.raises(exc):
        cca.fwd(q, off, k, v, phi="softmax", lse=lse)


@pytest.mark.parametrize("lse,exc", BAD_LSE)
def test_fwd_jagged_kv_rejects_bad_lse(lse, exc):
    q, off, kv_off, k, v = jagged()
    with pytest.raises(exc):
        cca.fwd_jagged_kv(q, off, kv_off, k, v, n_kv=4, phi="softmax", lse=lse)


@pytest.mark.parametrize("lse,exc", BAD_LSE)
def test_fwd_biased_rejects_bad_lse(lse, exc):
    q, off, k, v = base()
    with pytest.raises(exc):
        cca.fwd_biased(q, off, k, v, None, None, phi="softmax", lse=lse)


def test_jagged_and_biased_calls_reject_strided_q():
    q, off, kv_off, k, v = jagged()
    o = torch.zeros_like(q)
    lse = torch.zeros((T, H))
    with pytest.raises(ValueError, match="q"):
        cca.fwd_jagged_kv(strided_q(), off, kv_off, k, v, n_kv=4, phi="silu")
    with pytest.raises(ValueError, match="q"):
        cca.bwd_jagged_kv(strided_q(), off, kv_off, k, v, 4, o, lse, q, phi="silu")
    q, off, k, v = base()
    with pytest.raises(ValueError, match="q"):
        cca.fwd_biased(strided_q(), off, k, v, None, None, phi="silu")
    with pytest.raises(ValueError, match="q"):
        cca.bwd_biased(strided_q(), off, k, v, None, None, None, None, q, phi="silu")
    with pytest.raises(ValueError, match="q"):
        cca.GroupSpec(strided_q(), off, k, v, phi="silu").problem()


@pytest.mark.parametrize("which,bad,exc", [
    ("dq", torch.zeros((T, H, d + 1), dtype=bf), ValueError),
    ("dq", torch.zeros((T, H, d), dtype=torch.float32), TypeError),
    ("dk", torch.zeros((H, 7, d), dtype=bf).transpose(0, 1), ValueError),
    ("dv", torch.zeros((7, H, d - 1), dtype=bf), ValueError),
])
def test_bwd_jagged_kv_rejects_bad_outputs(which, bad, exc):
    q, off, kv_off, k, v = jagged()
    outs = {which: bad}
    with pytest.raises(exc):
        cca.bwd_jagged_kv(q, off, kv_off, k, v, 4, None, None, q, phi="silu", **outs)


def test_bwd_noalloc_rejects_bad_outputs():
    q, off, k, v = base()
    dk, dv = torch.zeros_like(k), torch.zeros_like(v)
    with pytest.raises(ValueError, match="dq"):
        cca.bwd_noalloc(q, off, k, v, None, None, q, torch.zeros((T, H, 8), dtype=bf), dk, dv, phi="silu")
    with pytest.raises(ValueError, match="dk"):
        cca.bwd_noalloc(q, off, k, v, None, None, q, torch.zeros_like(q), dk[:1], dv, phi="silu")
