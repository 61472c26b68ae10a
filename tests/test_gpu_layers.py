"""GPU parity of the Kunlun layer stack (GDPA + HSP pooling + self-attention per
layer, full and CompSkip schedules), driven through the C ABI, against the fp64
oracle: final states, pooled summaries, dX_0, weight gradients and seed
gradients.  Tolerance max|gpu - ref| / max|ref| <= 2e-2 per tensor (bf16)."""
import pytest
import torch

import gdpa_inputs as gi
from oracle import compskip_oracle as cso
from tests.gpu_helpers import TOL, max_abs_rel, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("schedule", ["full", "compskip"])
@pytest.mark.parametrize("d", [64, 128])
def test_layer_stack_matches_oracle(gdpa_lib, schedule, d):
    from context_cross_attention_amd.layers import KunlunLayers
    H, n, c, L, m, w = 2, 64, 64, 4, 8, 40
    inp = gi.make_layer_stack_inputs(("explicit", [130, 0, 257, 33, 600, 1]), 6, H, d, n, c, layers=L, m=m, seed=21)
    T = int(inp.offsets[-1])
    say(f"case: layer stack {schedule} T={T} H={H} d={d} n={n} c={c} L={L} m={m} window={w}")
    dev = "cuda"
    model = KunlunLayers(inp.offsets.to(dev), inp.ctx.to(dev), [x.to(dev) for x in inp.w_k],
                         [x.to(dev) for x in inp.w_v], [x.to(dev) for x in inp.seeds], H, n, T, w, schedule)
    xl, zs = model.forward(inp.x0.to(dev))
    gz = {l: inp.dz[l].to(dev) for l in zs}
    dx0, dwk, dwv, dsd = model.backward(inp.dx.to(dev), gz)
    torch.cuda.synchronize()
    recs, rxl, rzs = cso.forward(inp.x0, inp.offsets, inp.ctx, inp.w_k, inp.w_v, inp.seeds, H, n, w, schedule)
    rdx, rwk, rwv, rsd = cso.backward(recs, inp.offsets, inp.ctx, inp.w_k, inp.w_v, inp.seeds, H, n, w, schedule,
                                      inp.dx, {l: inp.dz[l] for l in rzs})
    assert set(zs) == set(rzs) and set(dwk) == set(rwk) and set(dsd) == set(rsd)
    errs = {"x_last": max_abs_rel(xl, rxl), "dx0": max_abs_rel(dx0, rdx)}
    errs.update({f"z{l}": max_abs_rel(zs[l], rzs[l]) for l in zs})
    errs.update({f"dwk{l}": max_abs_rel(dwk[l], rwk[l]) for l in dwk})
    errs.update({f"dwv{l}": max_abs_rel(dwv[l], rwv[l]) for l in dwv})
    errs.update({f"dseeds{l}": max_abs_rel(dsd[l], rsd[l]) for l in dsd})
    say("  errors:", {k: f"{e:.2e}" for k, e in errs.items()})
    for k, e in errs.items():
        assert e <= TOL["bf16"], (k, e)
