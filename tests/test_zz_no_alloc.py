"""The allocation-free backward (gdpa_bwd_noalloc) against gdpa_bwd with a caller
workspace: two calls in a row on one GPU, the second smaller, every score map
family and both residual-gradient modes."""
import pytest
import torch

import gdpa_inputs as gi
from tests.gpu_helpers import TOL, custom_config, device_inputs, max_abs_rel, say

pytestmark = pytest.mark.gpu

CASES = [
    # (lengths, H, d, n): the resident backward (d = 128, n <= 256), then a smaller batch on the
    # chunked backward with the query-tile dQ kernel (n > 256), which also uses the tile prefix sums.
    ([700, 0, 33, 1200, 129, 64], 4, 128, 256),
    ([90, 5, 300], 2, 64, 384),
]


@pytest.mark.parametrize("phi", ["silu", "softmax"])
def test_noalloc_equals_workspace_call(gdpa_lib, phi):
    cca = gdpa_lib
    for i, (lengths, H, d, n) in enumerate(CASES):
        cfg = custom_config(lengths, H, d, n, phi=phi)
        inp = gi.make_gdpa_inputs(cfg, seed=11 + i, sharp=True)
        q, off, k, v, do = device_inputs(inp)
        o, lse = cca.fwd(q, off, k, v, phi=phi)
        for residual in (False, True):
            say(f"noalloc call {i}: phi={phi} L={lengths} H={H} d={d} n={n} residual={residual}")
            ref = cca.bwd(q, off, k, v, o, lse, do, phi=phi, residual=residual)
            got = tuple(torch.full_like(t, float("nan")) for t in ref)
            cca.bwd_noalloc(q, off, k, v, o, lse, do, *got, phi=phi, residual=residual)
            torch.cuda.synchronize()
            for name, g, r in zip(("dq", "dk", "dv"), got, ref):
                err = max_abs_rel(g, r.float().cpu().double().numpy())
                assert err <= TOL["bf16"], (name, err)
                assert torch.equal(g, r), f"{name}: the two entry points run the same kernels"
