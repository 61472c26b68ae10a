"""GPU parity of seed pooling attention (through the C ABI) against the fp64 oracle:
1 to 32 seeds, samples from empty to several 1024-token chunks (ragged 128-token
blocks and 32-token wave slices), head widths 32 / 64 / 128.  Tolerance
max|gpu - ref| / max|ref| <= 2e-2 (bf16 inputs, fp32 accumulation)."""
import numpy as np
import pytest
import torch

import gdpa_inputs as gi
from oracle import pma_oracle as pma
from tests.gpu_helpers import TOL, max_abs_rel, say

pytestmark = pytest.mark.gpu

CASES = [
    # lengths, H, d, m
    ((300, 0, 1, 129, 517), 2, 128, 32),
    ((300, 0, 1, 129, 517), 2, 128, 7),
    ((2500, 31, 1024, 1025), 1, 128, 32),    # several chunks, chunk boundaries
    ((33, 4100), 2, 128, 1),
    ((260, 1500, 33), 2, 64, 16),
    ((260, 1500, 33), 3, 32, 32),
    ((0, 0), 2, 64, 5),                       # every sample empty
]


def run(cca, inp):
    seeds, k, v, do = (t.cuda() for t in (inp.seeds, inp.k, inp.v, inp.do))
    off = inp.offsets.cuda()
    o, lse = cca.pma_fwd(seeds, off, k, v)
    ds, dk, dv = cca.pma_bwd(seeds, off, k, v, o, lse, do)
    torch.cuda.synchronize()
    return o, lse, ds, dk, dv


def lse_errors(lse, lse_ref):
    g = lse.double().cpu().numpy()
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(g), empty), "empty samples must have lse = -inf"
    return max_abs_rel(np.where(empty, 0.0, g), np.where(empty, 0.0, lse_ref))


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"H{c[1]}d{c[2]}m{c[3]}L{max(c[0])}")
@pytest.mark.parametrize("sharp", [False, True], ids=["normal", "sharp"])
def test_pma_parity(gdpa_lib, case, sharp):
    cca = gdpa_lib
    lengths, H, d, m = case
    inp = gi.make_pma_inputs(("explicit", list(lengths)), len(lengths), H, d, m, seed=8, sharp=sharp)
    say(f"case: pma lengths={lengths} H={H} d={d} m={m} sharp={sharp}")
    o, lse, ds, dk, dv = run(cca, inp)
    o_ref, lse_ref = pma.pma_forward(inp.seeds, inp.offsets, inp.k, inp.v)
    ds_ref, dk_ref, dv_ref = pma.pma_backward(inp.seeds, inp.offsets, inp.k, inp.v, inp.do)
    errs = {"o": max_abs_rel(o, o_ref), "lse": lse_errors(lse, lse_ref), "dseeds": max_abs_rel(ds, ds_ref),
            "dk": max_abs_rel(dk, dk_ref), "dv": max_abs_rel(dv, dv_ref)}
    say("  errors:", {n_: f"{e:.2e}" for n_, e in errs.items()})
    for name, e in errs.items():
        assert e <= TOL["bf16"], (name, e)


def test_pma_single_token_and_constant_keys(gdpa_lib):
    # One-token samples pool to that token's V (exactly, after bf16 rounding of a
    # weight of 1); with K = 0 every seed pools the mean of V.
    cca = gdpa_lib
    inp = gi.make_pma_inputs(("explicit", [1, 1, 200]), 3, 2, 64, 32, seed=9, sharp=True)
    o, _, _, _, _ = run(cca, inp)
    v = inp.v
    assert torch.equal(o[0].cpu(), v[0].expand(32, 2, 64))
    assert torch.equal(o[1].cpu(), v[1].expand(32, 2, 64))
    k0 = torch.zeros_like(inp.k)
    seeds, off = inp.seeds.cuda(), inp.offsets.cuda()
    o2, lse2 = cca.pma_fwd(seeds, off, k0.cuda(), inp.v.cuda())
    torch.cuda.synchronize()
    mean = inp.v[2:].double().mean(0)
    assert float((o2[2].cpu().double() - mean).abs().max() / mean.abs().max()) <= TOL["bf16"]
    assert float((lse2[2].cpu() - np.log(200.0)).abs().max()) <= 1e-5


def test_pma_workspace_is_reusable(gdpa_lib):
    # A second call on the same workspace (partials left over from a larger batch)
    # gives the same results as a fresh one.
    cca = gdpa_lib
    big = gi.make_pma_inputs(("explicit", [3000, 2100, 40]), 3, 2, 128, 32, seed=10)
    small = gi.make_pma_inputs(("explicit", [1500, 7]), 2, 2, 128, 32, seed=11)
    ws = torch.empty(cca.pma_workspace_bytes(big.seeds, big.offsets, big.k, True), dtype=torch.uint8,
                     device="cuda")
    args_b = [t.cuda() for t in (big.seeds, big.offsets, big.k, big.v)]
    o, lse = cca.pma_fwd(*args_b, workspace=ws)
    cca.pma_bwd(*args_b, o, lse, big.do.cuda(), workspace=ws)
    args_s = [t.cuda() for t in (small.seeds, small.offsets, small.k, small.v)]
    o1, lse1 = cca.pma_fwd(*args_s, workspace=ws)
    g1 = cca.pma_bwd(*args_s, o1, lse1, small.do.cuda(), workspace=ws)
    o2, lse2 = cca.pma_fwd(*args_s)
    g2 = cca.pma_bwd(*args_s, o2, lse2, small.do.cuda())
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(lse1, lse2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_pma_rejects_bad_arguments(gdpa_lib):
    cca = gdpa_lib
    inp = gi.make_pma_inputs(("explicit", [5]), 1, 1, 64, 4, seed=12)
    seeds, k, v = (t.cuda() for t in (inp.seeds, inp.k, inp.v))
    off = inp.offsets.cuda()
    with pytest.raises(cca.GdpaError):
        cca.pma_fwd(seeds.float(), off, k.float(), v.float())      # fp32 not supported
    many = torch.zeros((33, 1, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cca.GdpaError):
        cca.pma_fwd(many, off, k, v)                               # more than 32 seeds
    odd = torch.zeros((4, 1, 48), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cca.GdpaError):
        cca.pma_fwd(odd, off, torch.zeros((5, 1, 48), dtype=torch.bfloat16, device="cuda"),
                    torch.zeros((5, 1, 48), dtype=torch.bfloat16, device="cuda"))


@pytest.mark.parametrize("case", [c for c in CASES if sum(c[0]) > 0], ids=lambda c: f"H{c[1]}d{c[2]}m{c[3]}L{max(c[0])}")
def test_pma_self_pooling_kv_sum(gdpa_lib, case):
    # A sequence pooled with itself (K = V = X, as HSP pools the token states): the
    # summed backward's dk is dK + dV of the oracle, and the seed gradient and the
    # forward are those of the plain call.
    cca = gdpa_lib
    lengths, H, d, m = case
    inp = gi.make_pma_inputs(("explicit", list(lengths)), len(lengths), H, d, m, seed=9, sharp=True)
    say(f"case: pma self-pooling lengths={lengths} H={H} d={d} m={m}")
    seeds, x, do, off = inp.seeds.cuda(), inp.k.cuda(), inp.do.cuda(), inp.offsets.cuda()
    o, lse = cca.pma_fwd(seeds, off, x, x)
    ds, dkv, dv = cca.pma_bwd(seeds, off, x, x, o, lse, do, kv_sum=True)
    ds2, dk2, dv2 = cca.pma_bwd(seeds, off, x, x, o, lse, do)
    torch.cuda.synchronize()
    assert dv is None and torch.equal(ds, ds2)
    ds_ref, dk_ref, dv_ref = pma.pma_backward(inp.seeds, inp.offsets, inp.k, inp.k, inp.do)
    err = max_abs_rel(dkv, dk_ref + dv_ref)
    say(f"  dK + dV error {err:.2e}")
    assert err <= TOL["bf16"]
    # One rounding of the two bf16 results' sum.
    assert torch.equal(dkv, (dk2.float() + dv2.float()).to(torch.bfloat16))
