"""GPU parity of weight generation (C W^T and its weight gradient) and of the
stacked residual layers (forward and backward) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import gdpa_inputs as gi
from oracle import gdpa_oracle as orc
from tests.gpu_helpers import TOL, max_abs_rel, say

pytestmark = pytest.mark.gpu


# Shapes: a single partial tile, the stacked workload's ctx width, degenerate sizes,
# ragged tiles with K below one k-step, and several m-tiles with a ragged K tail and
# ragged n (the persistent tile walk crosses tiles with a partial last k-step).
@pytest.mark.parametrize("B,c,cols", [(37, 64, 520), (128, 512, 1024), (1, 8, 8), (300, 40, 264),
                                      (1030, 200, 696), (513, 72, 2056)])
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


@pytest.mark.parametrize("phi", ["silu", "softmax"])
def test_stacked_layers_match_oracle(gdpa_lib, phi):
    from context_cross_attention_amd.stacked import StackedGdpa
    cfg = gi.small_config(gi.CONFIGS[5], batch=6, lengths=("explicit", [300, 0, 17, 129, 64, 1]),
                          n_kv=64, ctx_dim=64, layers=3)
    inp = gi.make_stacked_inputs(cfg, seed=11)
    T = int(inp.offsets[-1])
    say(f"case: stacked layers=3 T={T} H=8 d=128 n=64 c=64 phi={phi}")
    dev = "cuda"
    model = StackedGdpa(inp.offsets.to(dev), inp.ctx.to(dev), [w.to(dev) for w in inp.w_k],
                        [w.to(dev) for w in inp.w_v], cfg.heads, cfg.n_kv, T, phi=phi)
    x_last = model.forward(inp.x0.to(dev))
    dx0, dwk, dwv = model.backward(inp.do.to(dev))
    torch.cuda.synchronize()
    xs = orc.stacked_forward(inp.x0, inp.offsets, inp.ctx, inp.w_k, inp.w_v, cfg.heads, cfg.n_kv, phi)
    gx, gwk, gwv = orc.stacked_backward(xs, inp.offsets, inp.ctx, inp.w_k, inp.w_v, inp.do, cfg.heads,
                                        cfg.n_kv, phi)
    errs = {"x_last": max_abs_rel(x_last.reshape(T, -1), xs[-1]), "dx0": max_abs_rel(dx0.reshape(T, -1), gx)}
    for l in range(cfg.layers):
        errs[f"dwk{l}"] = max_abs_rel(dwk[l], gwk[l])
        errs[f"dwv{l}"] = max_abs_rel(dwv[l], gwv[l])
    say("  errors:", {k: f"{e:.2e}" for k, e in errs.items()})
    for k, e in errs.items():
        assert e <= TOL["bf16"], (k, e)


# The residual block forward (O and X + O in one pass): every forward kernel family.
BLOCK_SHAPES = [
    # lengths, H, d, n, dtype: resident (n d <= 32768), streaming, small head width, fp32
    ((300, 0, 17, 129), 4, 128, 100, "bf16"),
    ((150, 64, 9), 2, 128, 300, "bf16"),
    ((70, 1, 131), 2, 64, 40, "bf16"),
    ((64, 64, 64, 64), 2, 32, 64, "f32"),
]


@pytest.mark.parametrize("lengths,H,d,n,dtype", BLOCK_SHAPES)
@pytest.mark.parametrize("phi", ["softmax", "silu", "relu"])
def test_block_forward_keeps_o_and_sum(gdpa_lib, lengths, H, d, n, dtype, phi):
    from tests.gpu_helpers import custom_config, device_inputs
    cca = gdpa_lib
    cfg = custom_config(lengths, H, d, n, dtype=dtype, phi=phi, backward=False)
    inp = gi.make_gdpa_inputs(cfg, seed=21, sharp=(phi == "softmax"))
    q, off, k, v, _ = device_inputs(inp)
    say(f"case: block fwd L={lengths} H={H} d={d} n={n} {dtype} {phi}")
    o, y, lse = cca.fwd_block(q, off, k, v, phi=phi)
    o_plain, lse_plain = cca.fwd(q, off, k, v, phi=phi)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain), "O of the block call equals the plain forward's"
    if phi == "softmax":
        assert torch.equal(lse, lse_plain)
    o_ref, _ = orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, phi)
    tol = TOL[dtype]
    assert max_abs_rel(o, o_ref) <= tol
    assert max_abs_rel(y, orc.as_f64(inp.q) + o_ref) <= tol
    # y is O and X summed in fp32 then rounded once: within one rounding of o + x.
    yd = y.double().cpu().numpy()
    od = (o.double() + q.double()).cpu().numpy()
    assert np.abs(yd - od).max() <= (2.0 ** -7 if dtype == "bf16" else 1e-6) * max(np.abs(od).max(), 1e-30)
