"""GPU parity of sliding-window self-attention (through the C ABI) against the fp64
oracle: windows from 1 to longer than any sample, several 128-row forward tiles and
256-row backward chunks, ragged and empty samples, head widths 32 / 64 / 128.
Tolerance max|gpu - ref| / max|ref| <= 2e-2 (bf16 inputs, fp32 accumulation)."""
import numpy as np
import pytest
import torch

import gdpa_inputs as gi
from oracle import swa_oracle as swa
from tests.gpu_helpers import TOL, max_abs_rel, say

pytestmark = pytest.mark.gpu

CASES = [
    # lengths, H, d, window
    ((300, 0, 1, 129, 517), 2, 128, 64),
    ((300, 0, 1, 129, 517), 2, 128, 1),
    ((600, 40), 1, 128, 256),
    ((600, 40), 1, 128, 257),
    ((700, 3), 2, 128, 5000),       # window longer than every sample: causal attention
    ((260, 513, 33), 2, 64, 100),
    ((260, 513, 33), 3, 32, 37),
    ((1024,), 1, 128, 300),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"H{c[1]}d{c[2]}w{c[3]}L{max(c[0])}")
@pytest.mark.parametrize("sharp", [False, True], ids=["normal", "sharp"])
def test_swa_parity(gdpa_lib, case, sharp):
    cca = gdpa_lib
    lengths, H, d, w = case
    inp = gi.make_swa_inputs(("explicit", list(lengths)), len(lengths), H, d, seed=5, sharp=sharp)
    say(f"case: swa lengths={lengths} H={H} d={d} window={w} sharp={sharp}")
    q, k, v, do = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.do))
    off = inp.offsets.cuda()
    o, lse = cca.swa_fwd(q, off, k, v, w)
    dq, dk, dv = cca.swa_bwd(q, off, k, v, o, lse, do, w)
    torch.cuda.synchronize()
    o_ref, lse_ref = swa.swa_forward(inp.q, inp.offsets, inp.k, inp.v, w)
    dq_ref, dk_ref, dv_ref = swa.swa_backward(inp.q, inp.offsets, inp.k, inp.v, inp.do, w)
    errs = {"o": max_abs_rel(o, o_ref), "lse": max_abs_rel(lse, lse_ref), "dq": max_abs_rel(dq, dq_ref),
            "dk": max_abs_rel(dk, dk_ref), "dv": max_abs_rel(dv, dv_ref)}
    say("  errors:", {n_: f"{e:.2e}" for n_, e in errs.items()})
    for name, e in errs.items():
        assert e <= TOL["bf16"], (name, e)


def test_swa_window_one_is_identity_on_v(gdpa_lib):
    # Window 1: each token sees only itself, so O = V and dV = dO, dQ = dK = 0 exactly.
    cca = gdpa_lib
    inp = gi.make_swa_inputs(("explicit", [70, 0, 129]), 3, 2, 128, seed=6, sharp=True)
    q, k, v, do = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.do))
    off = inp.offsets.cuda()
    o, lse = cca.swa_fwd(q, off, k, v, 1)
    dq, dk, dv = cca.swa_bwd(q, off, k, v, o, lse, do, 1)
    torch.cuda.synchronize()
    assert torch.equal(o, v)
    assert torch.equal(dv, do)
    assert float(dq.float().abs().max()) <= 1e-2 and float(dk.float().abs().max()) <= 1e-2


def test_swa_rejects_bad_arguments(gdpa_lib):
    cca = gdpa_lib
    inp = gi.make_swa_inputs(("explicit", [5]), 1, 1, 64, seed=7)
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    off = inp.offsets.cuda()
    with pytest.raises(cca.GdpaError):
        cca.swa_fwd(q, off, k, v, 0)            # window < 1
    with pytest.raises(cca.GdpaError):
        cca.swa_fwd(q.float(), off, k.float(), v.float(), 4)   # fp32 not supported


BLOCK_CASES = [((300, 0, 1, 129, 517), 2, 128, 64), ((600, 40), 1, 128, 257), ((260, 513, 33), 2, 64, 100),
               ((260, 513, 33), 3, 32, 37)]


@pytest.mark.parametrize("case", BLOCK_CASES, ids=lambda c: f"H{c[1]}d{c[2]}w{c[3]}L{max(c[0])}")
def test_swa_block_parity(gdpa_lib, case):
    # Self-attention block with its residual: y = x + SWA(x, x, x) and
    # dx = dy + dQ + dK + dV, against the oracle composed the same way.
    cca = gdpa_lib
    lengths, H, d, w = case
    inp = gi.make_swa_inputs(("explicit", list(lengths)), len(lengths), H, d, seed=6)
    say(f"case: swa block lengths={lengths} H={H} d={d} window={w}")
    x, dy, off = inp.q.cuda(), inp.do.cuda(), inp.offsets.cuda()
    y, o, lse = cca.swa_block_fwd(x, off, w)
    dx = cca.swa_block_bwd(x, off, o, lse, dy, w)
    o2, lse2 = cca.swa_fwd(x, off, x, x, w)
    torch.cuda.synchronize()
    o_ref, lse_ref = swa.swa_forward(inp.q, inp.offsets, inp.q, inp.q, w)
    gq, gk, gv = swa.swa_backward(inp.q, inp.offsets, inp.q, inp.q, inp.do, w)
    y_ref = inp.q.double().numpy() + o_ref
    dx_ref = inp.do.double().numpy() + gq + gk + gv
    errs = {"y": max_abs_rel(y, y_ref), "o": max_abs_rel(o, o_ref), "lse": max_abs_rel(lse, lse_ref),
            "dx": max_abs_rel(dx, dx_ref)}
    say("  errors:", {n_: f"{e:.2e}" for n_, e in errs.items()})
    for name, e in errs.items():
        assert e <= TOL["bf16"], (name, e)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)   # the block's O is the plain call's
