"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Sizes span several 128-row forward tiles and 32-row backward steps, ragged
tails, empty samples, context lengths that are not multiples of the tile, and
context rows split over several work-groups.  Tolerance: max|gpu - ref| /
max|ref| <= 1e-4 for fp32 and 2e-2 for bf16 inputs with fp32 accumulation.
"""
import numpy as np
import pytest
import torch

import gdpa_inputs as gi
from oracle import gdpa_oracle as orc
from tests.gpu_helpers import TOL, custom_config, device_inputs, max_abs_rel, say

pytestmark = pytest.mark.gpu


def run_case(cca, cfg, phi, seed=0, sharp=False, scale=None, check_bwd=True):
    inp = gi.make_gdpa_inputs(cfg, seed=seed, sharp=sharp, with_grad=check_bwd)
    say(f"case: {cfg.name} phi={phi} seed={seed} sharp={sharp} T={inp.total_tokens}")
    q, off, k, v, do = device_inputs(inp)
    o, lse = cca.fwd(q, off, k, v, phi=phi, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, phi, scale)
    tol = TOL[cfg.dtype]
    errs = {"o": max_abs_rel(o, o_ref)}
    if phi == "softmax":
        errs["lse"] = max_abs_rel(lse, lse_ref)
    if check_bwd:
        dq, dk, dv = cca.bwd(q, off, k, v, o, lse, do, phi=phi, scale=scale)
        torch.cuda.synchronize()
        dq_ref, dk_ref, dv_ref = orc.gdpa_backward(inp.q, inp.offsets, inp.k, inp.v, inp.do, phi, scale)
        errs.update(dq=max_abs_rel(dq, dq_ref), dk=max_abs_rel(dk, dk_ref), dv=max_abs_rel(dv, dv_ref))
    say("  errors:", {k_: f"{e:.2e}" for k_, e in errs.items()})
    for name, e in errs.items():
        assert e <= tol, f"{name}: max-abs-rel {e:.3e} > {tol}"
    return errs


# fp32: the small fixed-length workload and ragged variants.
MORE_MAPS = ["relu", "gelu", "identity"]


@pytest.mark.parametrize("phi", ["softmax", "silu"] + MORE_MAPS)
def test_fp32_fixed_length_workload(gdpa_lib, phi):
    run_case(gdpa_lib, gi.small_config(gi.CONFIGS[1], backward=True), phi)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("phi", ["softmax", "silu"] + MORE_MAPS)
def test_fp32_ragged(gdpa_lib, d, phi):
    cfg = custom_config((0, 1, 37, 130), H=2, d=d, n=5, dtype="f32", phi=phi)
    run_case(gdpa_lib, cfg, phi, sharp=True)


# bf16 MFMA path.
BF16_SHAPES = [
    # lengths, H, d, n
    ((0, 1, 127, 128, 129, 300), 2, 128, 64),
    ((5, 260, 0, 33), 3, 128, 100),     # n not a multiple of the 64-row block
    ((200, 1, 77), 2, 128, 256),        # one 8-wave backward work-group per head
    ((150, 64, 9), 2, 128, 300),        # context rows over two backward work-groups (dQ per query tile)
    ((129, 3, 250), 4, 64, 256),
    ((70, 0, 131), 2, 64, 40),
    ((64, 200, 1), 2, 32, 64),
    ((33, 97), 1, 128, 1),              # a single context row
    # kernel-selection boundaries: largest resident forward context per head width
    # (n d = 32768) and one row more (streaming forward), backward chunk counts
    # with a one-row tail chunk
    ((300, 2, 77), 2, 64, 512),
    ((300, 2, 77), 2, 64, 513),
    ((100, 40), 1, 32, 1024),
    ((100, 40), 1, 32, 1025),
    ((130, 70), 2, 128, 129),
    ((40, 300), 1, 128, 2049),
]


@pytest.mark.parametrize("shape", BF16_SHAPES, ids=lambda s: f"H{s[1]}d{s[2]}n{s[3]}")
@pytest.mark.parametrize("phi", ["softmax", "silu"])
@pytest.mark.parametrize("sharp", [False, True], ids=["normal", "sharp"])
def test_bf16_parity(gdpa_lib, shape, phi, sharp):
    lengths, H, d, n = shape
    run_case(gdpa_lib, custom_config(lengths, H, d, n, phi=phi), phi, sharp=sharp)


@pytest.mark.parametrize("shape", BF16_SHAPES, ids=lambda s: f"H{s[1]}d{s[2]}n{s[3]}")
@pytest.mark.parametrize("phi", MORE_MAPS)
def test_bf16_parity_more_maps(gdpa_lib, shape, phi):
    # Scores of order one ("sharp" inputs), where the maps are far from linear; both the
    # resident-context kernels (d = 128, n <= 256) and the streaming ones are covered.
    lengths, H, d, n = shape
    run_case(gdpa_lib, custom_config(lengths, H, d, n, phi=phi), phi, sharp=True)


@pytest.mark.parametrize("phi", MORE_MAPS)
def test_bf16_more_maps_residual(gdpa_lib, phi):
    # Stacked-layer form (residual forward, residual dQ) on the resident-context kernels.
    cca = gdpa_lib
    cfg = custom_config((100, 0, 260, 7), H=2, d=128, n=200, phi=phi)
    inp = gi.make_gdpa_inputs(cfg, seed=3)
    q, off, k, v, do = device_inputs(inp)
    say(f"case: residual {phi}")
    o, _ = cca.fwd(q, off, k, v, phi=phi, residual=q)
    dx = do.clone()
    dq, dk, dv = cca.bwd(q, off, k, v, None, None, dx, phi=phi, dq=dx, residual=True)
    torch.cuda.synchronize()
    o_ref, _ = orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, phi)
    dq_ref, dk_ref, dv_ref = orc.gdpa_backward(inp.q, inp.offsets, inp.k, inp.v, inp.do, phi)
    errs = {"o": max_abs_rel(o.cpu(), o_ref + orc.as_f64(inp.q)),
            "dq": max_abs_rel(dq.cpu(), dq_ref + orc.as_f64(inp.do)),
            "dk": max_abs_rel(dk.cpu(), dk_ref), "dv": max_abs_rel(dv.cpu(), dv_ref)}
    say("  errors:", {n_: f"{e:.2e}" for n_, e in errs.items()})
    for name, e in errs.items():
        assert e <= TOL["bf16"], (phi, name, e)


def test_bf16_explicit_scale(gdpa_lib):
    cfg = custom_config((90, 140), H=2, d=128, n=128, phi="softmax")
    run_case(gdpa_lib, cfg, "softmax", scale=0.37, sharp=True)
    run_case(gdpa_lib, custom_config((90, 140), H=2, d=128, n=128, phi="silu"), "silu", scale=0.5)


@pytest.mark.parametrize("n", [200, 512], ids=["resident", "streaming"])
@pytest.mark.parametrize("scale", [-0.37, 0.0], ids=["negative", "zero"])
def test_bf16_softmax_nonpositive_scale(gdpa_lib, n, scale):
    # Any finite scale is accepted.  The forwards keep the softmax's running max in raw
    # Q.K units only for a positive scale (where the max commutes with it); a negative
    # scale turns the maximum into a minimum and a zero scale makes every score 0 (the
    # uniform average, LSE = ln n).  Both forward kernels (resident context, n <= 256
    # at d = 128, and the streaming one) and the backward are checked.
    cfg = custom_config((90, 140, 7), H=2, d=128, n=n, phi="softmax")
    run_case(gdpa_lib, cfg, "softmax", scale=scale, sharp=True)


def very_negative_scores(base, d, seed):
    """Q and K of `base` replaced so that every score is below about -100: every query is
    40 u (plus a little noise) and every key row -40 u + w_j, u the unit vector along
    (1, ..., 1) and w_j with entries N(0, 1600 / d).  The shared key component is no
    larger than the varying one (|w_j| is about 40), so dQ stays well conditioned
    against the bf16 rounding of dS (the shared part cancels from dQ only exactly)."""
    import dataclasses
    rng = np.random.default_rng(seed)
    u = np.full(d, 1.0 / np.sqrt(d))
    H = base.q.shape[1]
    q = 40 * u + 0.05 * rng.standard_normal((base.q.shape[0], H, d))
    k = -40 * u + (40 / np.sqrt(d)) * rng.standard_normal(tuple(base.k.shape))
    return dataclasses.replace(base, q=torch.from_numpy(q).to(torch.bfloat16),
                               k=torch.from_numpy(k).to(torch.bfloat16))


@pytest.mark.parametrize("d,n", [(128, 100), (64, 100), (128, 300)],
                         ids=["one-work-group", "key-chunk-with-dq", "key-chunk-and-query-tile"])
def test_bf16_softmax_all_scores_very_negative(gdpa_lib, d, n):
    # Every score of every token below about -100, so the row LSE is too and exp(-LSE)
    # overflows fp32.  The backward kernels compute P for context rows past n (zero K and
    # V rows, score 0) as exp(-LSE); they must keep it finite there (no inf * 0 in dQ),
    # whatever the path: the one-work-group backward (d = 128, n <= 256), the key-chunk
    # kernel with its own dQ (d = 64), and the key-chunk kernel plus the query-tile dQ
    # kernel (n = 300).
    cfg = custom_config((70, 33, 130), H=2, d=d, n=n, phi="softmax")
    inp = very_negative_scores(gi.make_gdpa_inputs(cfg, seed=5, with_grad=True), d, seed=6)
    say(f"case: very negative scores d={d} n={n} T={inp.total_tokens}")
    qd, off, kd, vd, do = device_inputs(inp)
    o, lse = gdpa_lib.fwd(qd, off, kd, vd, phi="softmax")
    dq, dk, dv = gdpa_lib.bwd(qd, off, kd, vd, o, lse, do, phi="softmax")
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, "softmax")
    assert float(np.nanmax(lse_ref)) < -90.0  # the premise of the case
    refs = dict(zip(("dq", "dk", "dv"), orc.gdpa_backward(inp.q, inp.offsets, inp.k, inp.v, inp.do, "softmax")))
    errs = {"o": max_abs_rel(o, o_ref), "lse": max_abs_rel(lse, lse_ref)}
    errs.update({name: max_abs_rel(got, refs[name]) for name, got in (("dq", dq), ("dk", dk), ("dv", dv))})
    say("  errors:", {k_: f"{e:.2e}" for k_, e in errs.items()})
    for t in (o, lse, dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    for name, e in errs.items():
        assert e <= TOL["bf16"], f"{name}: max-abs-rel {e:.3e}"


@pytest.mark.parametrize("dtype,d,n", [("bf16", 64, 96), ("f32", 64, 96), ("bf16", 128, 200)])
@pytest.mark.parametrize("mode", ["accumulate", "residual"])
def test_residual_and_accumulated_dq(gdpa_lib, dtype, d, n, mode):
    """O = X + GDPA(X), and dX = dO + dQ written in place over dO, either by
    accumulating into a dq buffer that already holds dO or by the residual flag."""
    cca = gdpa_lib
    cfg = custom_config((100, 0, 260, 7), H=2, d=d, n=n, dtype=dtype, phi="silu")
    inp = gi.make_gdpa_inputs(cfg, seed=3)
    q, off, k, v, do = device_inputs(inp)
    o, _ = cca.fwd(q, off, k, v, phi="silu", residual=q)
    o_ref, _ = orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, "silu")
    o_ref = o_ref + orc.as_f64(inp.q)
    assert max_abs_rel(o, o_ref) <= TOL[dtype]
    dq_ref, dk_ref, dv_ref = orc.gdpa_backward(inp.q, inp.offsets, inp.k, inp.v, inp.do, "silu")
    dx = do.clone()
    if mode == "accumulate":
        dq, dk, dv = cca.bwd(q, off, k, v, None, None, dx, phi="silu", dq=dx, accumulate_dq=True)
    else:
        dq, dk, dv = cca.bwd(q, off, k, v, None, None, dx, phi="silu", dq=dx, residual=True)
    torch.cuda.synchronize()
    assert dq.data_ptr() == dx.data_ptr()
    assert max_abs_rel(dx, dq_ref + orc.as_f64(inp.do)) <= TOL[dtype]
    assert max_abs_rel(dk, dk_ref) <= TOL[dtype] and max_abs_rel(dv, dv_ref) <= TOL[dtype]


def test_accumulated_dq_split_context(gdpa_lib):
    """Accumulating dQ when the context spans two key-chunk work-groups: dQ then comes
    from the query-tile kernel, which adds the existing dq in its epilogue."""
    cca = gdpa_lib
    cfg = custom_config((100, 40), H=2, d=128, n=300, phi="softmax")
    inp = gi.make_gdpa_inputs(cfg, seed=4, sharp=True)
    q, off, k, v, do = device_inputs(inp)
    o, lse = cca.fwd(q, off, k, v, phi="softmax")
    dx = do.clone()
    cca.bwd(q, off, k, v, o, lse, dx, phi="softmax", dq=dx, accumulate_dq=True)
    torch.cuda.synchronize()
    dq_ref, _, _ = orc.gdpa_backward(inp.q, inp.offsets, inp.k, inp.v, inp.do, "softmax")
    assert max_abs_rel(dx, dq_ref + orc.as_f64(inp.do)) <= TOL["bf16"]


def test_empty_batch_and_empty_samples(gdpa_lib):
    cca = gdpa_lib
    cfg = custom_config((0, 0, 0), H=2, d=128, n=64, phi="softmax")
    inp = gi.make_gdpa_inputs(cfg, seed=5)
    q, off, k, v, do = device_inputs(inp)
    o, lse = cca.fwd(q, off, k, v, phi="softmax")
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(v, 7.0)
    cca.bwd(q, off, k, v, o, lse, do, phi="softmax", dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert torch.all(dk == 0) and torch.all(dv == 0)


def test_softmax_rows_sum_to_one_on_gpu(gdpa_lib):
    """With V = 1 every output row is exactly 1 up to bf16 rounding of P."""
    cca = gdpa_lib
    cfg = custom_config((300, 17), H=2, d=128, n=200, phi="softmax")
    inp = gi.make_gdpa_inputs(cfg, seed=6, sharp=True, with_grad=False)
    q, off, k, v, _ = device_inputs(inp)
    o, _ = cca.fwd(q, off, k, torch.ones_like(v), phi="softmax")
    torch.cuda.synchronize()
    assert float((o.float() - 1).abs().max()) <= 1e-2


def test_repeat_runs_stable(gdpa_lib):
    """Forward is deterministic; backward without atomics is deterministic too."""
    cca = gdpa_lib
    cfg = custom_config((300, 5, 129), H=2, d=128, n=256, phi="silu")
    inp = gi.make_gdpa_inputs(cfg, seed=7)
    q, off, k, v, do = device_inputs(inp)
    o1, _ = cca.fwd(q, off, k, v, phi="silu")
    o2, _ = cca.fwd(q, off, k, v, phi="silu")
    g1 = cca.bwd(q, off, k, v, None, None, do, phi="silu")
    g2 = cca.bwd(q, off, k, v, None, None, do, phi="silu")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_golden_tiny_cases(gdpa_lib):
    """The frozen tiny fixtures (oracle outputs), run on the fp32 path."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "tiny_cases.json")) as f:
        cases = json.load(f)["cases"]
    cca = gdpa_lib
    # The fixtures use tiny head widths (2, 4); they run on the fp32 path padded with zero
    # columns to d = 32, which leaves every score and every output column unchanged.
    for c in cases:
        q, k, v, do = (torch.tensor(np.array(c[x]), dtype=torch.float32) for x in ("q", "k", "v", "do"))
        d = c["d"]
        pad = lambda t: torch.nn.functional.pad(t, (0, 32 - d)).contiguous().cuda()  # noqa: E731
        off = torch.tensor(c["offsets"], dtype=torch.int32).cuda()
        scale = c["scale"] if c["scale"] is not None else orc.default_scale(c["phi"], d)
        o, lse = cca.fwd(pad(q), off, pad(k), pad(v), phi=c["phi"], scale=scale)
        dq, dk, dv = cca.bwd(pad(q), off, pad(k), pad(v), o, lse, pad(do), phi=c["phi"], scale=scale)
        torch.cuda.synchronize()
        assert max_abs_rel(o[..., :d], np.array(c["o"])) <= 1e-5
        assert max_abs_rel(dq[..., :d], np.array(c["dq"])) <= 1e-5
        assert max_abs_rel(dk[..., :d], np.array(c["dk"])) <= 1e-5
        assert max_abs_rel(dv[..., :d], np.array(c["dv"])) <= 1e-5
