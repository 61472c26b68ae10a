"""GPU parity of weight generation (C W^T and its weight gradient) and of the
stacked residual layers (forward and backward) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import gdpa_inputs as gi
from oracle import gdpa_oracle as orc
from tests.gpu_helpers import TOL, max_abs_rel, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,c,cols", [(37, 64, 520), (128, 512, 1024), (1, 8, 8), (300, 40, 264)])
def test_weightgen_gemms(gdpa_lib, B, c, cols):
    cca = gdpa_lib
    rng = np.random.default_rng(B + c + cols)
    ctx = torch.from_numpy(rng.standard_normal((B, c), dtype=np.float32)).bfloat16()
    w = torch.from_numpy(rng.standard_normal((cols, c), dtype=np.float32) / np.sqrt(c)).bfloat16()
    g = torch.from_numpy(rng.standard_normal((B, cols), dtype=np.float32)).bfloat16()
    say(f"case: weightgen B={B} c={c} cols={cols}")
    out = cca.weightgen_fwd(ctx.cuda(), w.cuda())
    dw = cca.weightgen_bwd_w(ctx.cuda(), g.cuda())
    torch.cuda.synchronize()
    ref = orc.as_f64(ctx) @ orc.as_f64(w).T
    assert max_abs_rel(out, ref) <= TOL["bf16"]
    assert max_abs_rel(dw, orc.weight_gradient(ctx, g)) <= TOL["bf16"]


def test_stacked_layers_match_oracle(gdpa_lib):
    from context_cross_attention_amd.stacked import StackedGdpa
    cfg = gi.small_config(gi.CONFIGS[5], batch=6, lengths=("explicit", [300, 0, 17, 129, 64, 1]),
                          n_kv=64, ctx_dim=64, layers=3)
    inp = gi.make_stacked_inputs(cfg, seed=11)
    T = int(inp.offsets[-1])
    say(f"case: stacked layers=3 T={T} H=8 d=128 n=64 c=64")
    dev = "cuda"
    model = StackedGdpa(inp.offsets.to(dev), inp.ctx.to(dev), [w.to(dev) for w in inp.w_k],
                        [w.to(dev) for w in inp.w_v], cfg.heads, cfg.n_kv, T, phi="silu")
    x_last = model.forward(inp.x0.to(dev))
    dx0, dwk, dwv = model.backward(inp.do.to(dev))
    torch.cuda.synchronize()
    xs = orc.stacked_forward(inp.x0, inp.offsets, inp.ctx, inp.w_k, inp.w_v, cfg.heads, cfg.n_kv, "silu")
    gx, gwk, gwv = orc.stacked_backward(xs, inp.offsets, inp.ctx, inp.w_k, inp.w_v, inp.do, cfg.heads,
                                        cfg.n_kv, "silu")
    errs = {"x_last": max_abs_rel(x_last.reshape(T, -1), xs[-1]), "dx0": max_abs_rel(dx0.reshape(T, -1), gx)}
    for l in range(cfg.layers):
        errs[f"dwk{l}"] = max_abs_rel(dwk[l], gwk[l])
        errs[f"dwv{l}"] = max_abs_rel(dwv[l], gwv[l])
    say("  errors:", {k: f"{e:.2e}" for k, e in errs.items()})
    for k, e in errs.items():
        assert e <= TOL["bf16"], (k, e)
