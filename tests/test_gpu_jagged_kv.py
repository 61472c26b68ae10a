"""GPU parity of GDPA with a jagged context (each sample owns kv_offsets[b+1] -
kv_offsets[b] context rows) against the fp64 oracle, through the C ABI: the
resident kernels (n * d <= 32768), the streaming forward, the chunked backward
with the query-tile dQ kernel, and the fp32 kernels; counts from 1 to beyond one
backward chunk, empty token samples, several score maps.  Tolerance
max|gpu - ref| / max|ref| <= 2e-2 (bf16), 1e-4 (fp32)."""
import numpy as np
import pytest
import torch

import gdpa_inputs as gi
from oracle import gdpa_oracle as orc
from tests.gpu_helpers import TOL, max_abs_rel, say

pytestmark = pytest.mark.gpu

CASES = [
    # token lengths, context counts, H, d, dtype
    ((300, 0, 129, 517, 64), (1, 7, 256, 100, 64), 2, 128, "bf16"),    # resident fwd + bwd
    ((200, 77, 0, 160), (512, 3, 40, 300), 2, 64, "bf16"),              # resident fwd, chunked bwd
    ((260, 130, 33), (1024, 300, 1), 1, 128, "bf16"),                   # streaming fwd, split dQ
    ((150, 90), (700, 65), 2, 32, "bf16"),                              # d = 32
    ((40, 0, 23), (5, 64, 17), 2, 32, "f32"),                           # fp32 kernels
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[4]}H{c[2]}d{c[3]}n{max(c[1])}")
@pytest.mark.parametrize("phi", ["softmax", "silu", "gelu"])
def test_jagged_kv_parity(gdpa_lib, case, phi):
    cca = gdpa_lib
    lengths, counts, H, d, dtype = case
    inp = gi.make_jagged_kv_inputs(("explicit", list(lengths)), ("explicit", list(counts)), len(lengths), H, d,
                                   seed=13, sharp=(phi == "softmax"), dtype=dtype)
    say(f"case: jagged kv lengths={lengths} counts={counts} H={H} d={d} {dtype} phi={phi}")
    q, k, v, do = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.do))
    off, ko = inp.offsets.cuda(), inp.kv_offsets.cuda()
    o, lse = cca.fwd_jagged_kv(q, off, ko, k, v, inp.n_kv, phi=phi)
    dq, dk, dv = cca.bwd_jagged_kv(q, off, ko, k, v, inp.n_kv, o, lse, do, phi=phi)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, phi, kv_offsets=inp.kv_offsets)
    dq_ref, dk_ref, dv_ref = orc.gdpa_backward(inp.q, inp.offsets, inp.k, inp.v, inp.do, phi,
                                               kv_offsets=inp.kv_offsets)
    errs = {"o": max_abs_rel(o, o_ref), "dq": max_abs_rel(dq, dq_ref), "dk": max_abs_rel(dk, dk_ref),
            "dv": max_abs_rel(dv, dv_ref)}
    if lse is not None:
        errs["lse"] = max_abs_rel(lse, lse_ref)
    say("  errors:", {n_: f"{e:.2e}" for n_, e in errs.items()})
    for name, e in errs.items():
        assert e <= TOL[dtype], (name, e)


def test_jagged_kv_equal_counts_match_dense(gdpa_lib):
    # With every sample owning n rows the jagged call is the dense call on the same memory.
    cca = gdpa_lib
    inp = gi.make_jagged_kv_inputs(("explicit", [90, 0, 200]), ("explicit", [64, 64, 64]), 3, 2, 128, seed=14)
    q, k, v, do = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.do))
    off, ko = inp.offsets.cuda(), inp.kv_offsets.cuda()
    for phi in ("softmax", "silu"):
        o1, l1 = cca.fwd_jagged_kv(q, off, ko, k, v, 64, phi=phi)
        g1 = cca.bwd_jagged_kv(q, off, ko, k, v, 64, o1, l1, do, phi=phi)
        kd, vd = k.view(3, 64, 2, 128), v.view(3, 64, 2, 128)
        o2, l2 = cca.fwd(q, off, kd, vd, phi=phi)
        g2 = cca.bwd(q, off, kd, vd, o2, l2, do, phi=phi)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
        for a, b in zip(g1, g2):
            assert torch.equal(a.reshape(-1), b.reshape(-1))


def test_check_kv_offsets_host(gdpa_lib):
    cca = gdpa_lib
    assert cca.check_kv_offsets([0, 3, 4, 10], 6)
    assert not cca.check_kv_offsets([0, 3, 3, 10], 8)     # a sample without context rows
    assert not cca.check_kv_offsets([0, 3, 4, 10], 5)     # more rows than n_kv
    assert not cca.check_kv_offsets([1, 3, 4], 5)         # does not start at 0
