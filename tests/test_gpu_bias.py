"""GPU parity of GDPA with FFN biases, O = phi(scale Q K^T + b_s) V + b_o, against
the fp64 oracle through the C ABI: O, LSE, dQ, dK, dV and both bias gradients,
over the resident kernels, the streaming forward, the chunked backward with the
query-tile dQ kernel and the fp32 kernels, with a dense and a jagged context,
with either bias alone.  Tolerance max|gpu - ref| / max|ref| <= 2e-2 (bf16),
1e-4 (fp32)."""
import pytest
import torch

import gdpa_inputs as gi
from oracle import gdpa_oracle as orc
from tests.gpu_helpers import TOL, max_abs_rel, say

pytestmark = pytest.mark.gpu

CASES = [
    # token lengths, context counts (None: dense n), n dense, H, d, dtype
    ((300, 0, 129, 517), None, 128, 2, 128, "bf16"),                  # resident fwd + bwd, dense
    ((300, 0, 129, 517, 64), (1, 7, 256, 100, 64), 0, 2, 128, "bf16"),  # resident, jagged
    ((200, 77, 0, 160), None, 512, 2, 64, "bf16"),                    # resident fwd, chunked bwd
    ((200, 77, 0, 160), (512, 3, 40, 300), 0, 2, 64, "bf16"),
    ((260, 130, 33), None, 1024, 1, 128, "bf16"),                     # streaming fwd, split dQ
    ((260, 130, 33), (1024, 300, 1), 0, 1, 128, "bf16"),
    ((150, 90), (700, 65), 0, 2, 32, "bf16"),                         # d = 32
    ((40, 0, 23), None, 20, 2, 32, "f32"),                            # fp32 kernels
    ((40, 0, 23), (5, 64, 17), 0, 2, 32, "f32"),
]


def _inputs(lengths, counts, n, H, d, dtype, phi, seed, out_scale=None):
    B = len(lengths)
    spec = ("explicit", list(counts)) if counts is not None else ("explicit", [n] * B)
    inp = gi.make_jagged_kv_inputs(("explicit", list(lengths)), spec, B, H, d, seed=seed,
                                   sharp=(phi == "softmax"), dtype=dtype)
    if counts is None:
        k = inp.k.view(B, n, H, d)
        v = inp.v.view(B, n, H, d)
        sb, ob = gi.draw_ffn_biases(seed + 1, (B, n, H), B, H, d, out_scale)
        return inp, k, v, None, n, sb, ob
    sb, ob = gi.draw_ffn_biases(seed + 1, (inp.k.shape[0], H), B, H, d, out_scale)
    return inp, inp.k, inp.v, inp.kv_offsets, inp.n_kv, sb, ob


def _run(cca, inp, k, v, ko, n_kv, sb, ob, phi):
    q, do, off = inp.q.cuda(), inp.do.cuda(), inp.offsets.cuda()
    kc, vc = k.cuda(), v.cuda()
    koc = None if ko is None else ko.cuda()
    sbc = None if sb is None else sb.cuda()
    obc = None if ob is None else ob.cuda()
    o, lse = cca.fwd_biased(q, off, kc, vc, sbc, obc, phi=phi, kv_offsets=koc, n_kv=n_kv)
    grads = cca.bwd_biased(q, off, kc, vc, sbc, obc, o, lse, do, phi=phi, kv_offsets=koc, n_kv=n_kv)
    torch.cuda.synchronize()
    return o, lse, grads


def _ref(inp, k, v, ko, sb, ob, phi):
    o, lse = orc.gdpa_forward(inp.q, inp.offsets, k, v, phi, kv_offsets=ko, score_bias=sb, out_bias=ob)
    g = orc.gdpa_backward(inp.q, inp.offsets, k, v, inp.do, phi, kv_offsets=ko, score_bias=sb, bias_grads=True)
    return o, lse, g


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[5]}H{c[3]}d{c[4]}n{c[2] or max(c[1])}"
                         + ("j" if c[1] else ""))
@pytest.mark.parametrize("phi", ["softmax", "silu", "gelu"])
def test_bias_parity(gdpa_lib, case, phi):
    lengths, counts, n, H, d, dtype = case
    inp, k, v, ko, n_kv, sb, ob = _inputs(lengths, counts, n, H, d, dtype, phi, seed=21)
    say(f"case: biased lengths={lengths} counts={counts} n={n_kv} H={H} d={d} {dtype} phi={phi}")
    o, lse, (dq, dk, dv, dsb, dob) = _run(gdpa_lib, inp, k, v, ko, n_kv, sb, ob, phi)
    o_r, lse_r, (dq_r, dk_r, dv_r, dsb_r, dob_r) = _ref(inp, k, v, ko, sb, ob, phi)
    errs = {"o": max_abs_rel(o, o_r), "dq": max_abs_rel(dq, dq_r), "dk": max_abs_rel(dk, dk_r),
            "dv": max_abs_rel(dv, dv_r), "dsb": max_abs_rel(dsb, dsb_r), "dob": max_abs_rel(dob, dob_r)}
    if lse is not None:
        errs["lse"] = max_abs_rel(lse, lse_r)
    say("  errors:", {n_: f"{e:.2e}" for n_, e in errs.items()})
    for name, e in errs.items():
        assert e <= TOL[dtype], (name, e)


@pytest.mark.parametrize("case", [((40, 0, 23), (5, 64, 17), 0, 2, 32, "f32"),
                                  ((300, 0, 129, 517), None, 128, 2, 128, "bf16"),
                                  ((260, 130, 33), (1024, 300, 1), 0, 1, 128, "bf16")],
                         ids=["f32", "bf16-resident", "bf16-split-dq"])
def test_large_out_bias(gdpa_lib, case):
    # Softmax with an output bias far larger than P V: the row term sum (P V) dO keeps
    # its accuracy (fp32: from O - b_o; bf16: from P V recomputed without the bias).
    lengths, counts, n, H, d, dtype = case
    inp, k, v, ko, n_kv, sb, ob = _inputs(lengths, counts, n, H, d, dtype, "softmax", seed=24, out_scale=4.0)
    o, lse, (dq, dk, dv, dsb, dob) = _run(gdpa_lib, inp, k, v, ko, n_kv, sb, ob, "softmax")
    o_r, lse_r, (dq_r, dk_r, dv_r, dsb_r, dob_r) = _ref(inp, k, v, ko, sb, ob, "softmax")
    errs = {"o": max_abs_rel(o, o_r), "dq": max_abs_rel(dq, dq_r), "dk": max_abs_rel(dk, dk_r),
            "dv": max_abs_rel(dv, dv_r), "dsb": max_abs_rel(dsb, dsb_r), "dob": max_abs_rel(dob, dob_r)}
    say(f"case: large output bias {dtype} n={n_kv}", {n_: f"{e:.2e}" for n_, e in errs.items()})
    for name, e in errs.items():
        assert e <= TOL[dtype], (name, e)


@pytest.mark.parametrize("which", ["score", "out"])
@pytest.mark.parametrize("phi", ["softmax", "silu"])
def test_single_bias(gdpa_lib, which, phi):
    # Either bias alone; the other pointer is null.
    inp, k, v, ko, n_kv, sb, ob = _inputs((300, 0, 129, 517), None, 128, 2, 128, "bf16", phi, seed=22)
    sb, ob = (sb, None) if which == "score" else (None, ob)
    o, lse, (dq, dk, dv, dsb, dob) = _run(gdpa_lib, inp, k, v, ko, n_kv, sb, ob, phi)
    o_r, lse_r, (dq_r, dk_r, dv_r, dsb_r, dob_r) = _ref(inp, k, v, ko, sb, ob, phi)
    errs = {"o": max_abs_rel(o, o_r), "dq": max_abs_rel(dq, dq_r), "dk": max_abs_rel(dk, dk_r),
            "dv": max_abs_rel(dv, dv_r), "dsb": max_abs_rel(dsb, dsb_r), "dob": max_abs_rel(dob, dob_r)}
    say(f"case: single {which} bias phi={phi}", {n_: f"{e:.2e}" for n_, e in errs.items()})
    for name, e in errs.items():
        assert e <= TOL["bf16"], (name, e)


def test_zero_bias_matches_unbiased(gdpa_lib):
    # Zero biases give the unbiased results.
    cca = gdpa_lib
    inp, k, v, ko, n_kv, sb, ob = _inputs((300, 0, 129, 517), None, 128, 2, 128, "bf16", "silu", seed=23)
    sb.zero_()
    ob.zero_()
    for phi in ("softmax", "silu"):
        o1, l1, g1 = _run(cca, inp, k, v, ko, n_kv, sb, ob, phi)
        q, do, off = inp.q.cuda(), inp.do.cuda(), inp.offsets.cuda()
        o2, l2 = cca.fwd(q, off, k.cuda(), v.cuda(), phi=phi)
        g2 = cca.bwd(q, off, k.cuda(), v.cuda(), o2, l2, do, phi=phi)
        torch.cuda.synchronize()
        # Adding a zero bias is exact, so all but a rare contraction-order difference
        # (one bf16 ulp) must agree bit for bit.
        for a, b in zip((o1,) + tuple(g1[:3]), (o2,) + tuple(g2)):
            same = (a == b).float().mean().item()
            assert same >= 0.999 and max_abs_rel(a, b.double().cpu().numpy()) <= 1e-2, same
