"""GPU checks of the grouped launch (event-level personalisation: one GDPA problem
per event type, each with its own heads, head width, context size, score map and
batch) through the C ABI: every group against the fp64 oracle; the grouped call
equal, bit for bit, to the same problems called one by one (the groups share no
memory and run the same kernels); replays of a captured HIP graph of the grouped
call equal to the eager call.  Tolerance max|gpu - ref| / max|ref| <= 2e-2
(bf16), 1e-4 (fp32)."""
import pytest
import torch

import gdpa_inputs as gi
from oracle import gdpa_oracle as orc
from tests.gpu_helpers import TOL, max_abs_rel, say

pytestmark = pytest.mark.gpu

PHIS = {"click": "softmax", "impression": "silu", "conversion": "gelu"}


def _specs(cca, events, phis):
    specs, dos = [], []
    for name, inp in events.items():
        specs.append(cca.GroupSpec(inp.q.cuda(), inp.offsets.cuda(), inp.k.cuda(), inp.v.cuda(), phi=phis[name]))
        dos.append(inp.do.cuda())
    return specs, dos


def test_grouped_parity(gdpa_lib):
    cca = gdpa_lib
    events = gi.make_event_inputs(seed=31, shrink=16, sharp=True)
    specs, dos = _specs(cca, events, PHIS)
    refs = [(inp, PHIS[name]) for name, inp in events.items()]
    # A jagged-context group and an fp32 group in the same call.
    jag = gi.make_jagged_kv_inputs(("explicit", [90, 0, 200]), ("explicit", [5, 64, 300]), 3, 2, 64, seed=32)
    specs.append(cca.GroupSpec(jag.q.cuda(), jag.offsets.cuda(), jag.k.cuda(), jag.v.cuda(), phi="silu",
                               kv_offsets=jag.kv_offsets.cuda(), n_kv=jag.n_kv))
    dos.append(jag.do.cuda())
    f32 = gi.make_gdpa_inputs(gi.CONFIGS[1], seed=33, sharp=True, with_grad=True)
    specs.append(cca.GroupSpec(f32.q.cuda(), f32.offsets.cuda(), f32.k.cuda(), f32.v.cuda(), phi="softmax"))
    dos.append(f32.do.cuda())
    outs = cca.fwd_grouped(specs)
    grads = cca.bwd_grouped(specs, outs, dos)
    torch.cuda.synchronize()
    cases = [(inp.q, inp.offsets, inp.k, inp.v, inp.do, phi, None, "bf16") for inp, phi in refs]
    cases.append((jag.q, jag.offsets, jag.k, jag.v, jag.do, "silu", jag.kv_offsets, "bf16"))
    cases.append((f32.q, f32.offsets, f32.k, f32.v, f32.do, "softmax", None, "f32"))
    for i, (q, off, k, v, do, phi, ko, dt) in enumerate(cases):
        o_r, lse_r = orc.gdpa_forward(q, off, k, v, phi, kv_offsets=ko)
        g_r = orc.gdpa_backward(q, off, k, v, do, phi, kv_offsets=ko)
        (o, lse), (dq, dk, dv) = outs[i], grads[i]
        errs = {"o": max_abs_rel(o, o_r), "dq": max_abs_rel(dq, g_r[0]), "dk": max_abs_rel(dk, g_r[1]),
                "dv": max_abs_rel(dv, g_r[2])}
        if lse is not None:
            errs["lse"] = max_abs_rel(lse, lse_r)
        say(f"group {i}: T={q.shape[0]} H={q.shape[1]} d={q.shape[2]} phi={phi} {dt}",
            {n_: f"{e:.2e}" for n_, e in errs.items()})
        for name, e in errs.items():
            assert e <= TOL[dt], (i, name, e)


def test_grouped_equals_single_calls(gdpa_lib):
    cca = gdpa_lib
    events = gi.make_event_inputs(seed=0)
    say("case: full-size event mix", {k: tuple(v.q.shape) for k, v in events.items()})
    specs, dos = _specs(cca, events, PHIS)
    outs = cca.fwd_grouped(specs)
    grads = cca.bwd_grouped(specs, outs, dos)
    for i, sp in enumerate(specs):
        o, lse = cca.fwd(sp.q, sp.offsets, sp.k, sp.v, phi=sp.phi)
        g = cca.bwd(sp.q, sp.offsets, sp.k, sp.v, o, lse, dos[i], phi=sp.phi)
        torch.cuda.synchronize()
        assert torch.equal(outs[i][0], o), i
        if lse is not None:
            assert torch.equal(outs[i][1], lse), i
        for a, b in zip(grads[i], g):
            assert torch.equal(a, b), i


def test_grouped_graph_replays(gdpa_lib):
    cca = gdpa_lib
    events = gi.make_event_inputs(seed=34, shrink=8)
    specs, dos = _specs(cca, events, PHIS)
    eager_o = cca.fwd_grouped(specs)
    eager_g = cca.bwd_grouped(specs, eager_o, dos)
    torch.cuda.synchronize()
    outs = [(torch.empty_like(o), None if l is None else torch.empty_like(l)) for o, l in eager_o]
    grads = [tuple(torch.empty_like(t) for t in g) for g in eager_g]
    ws_f = torch.empty(cca.grouped_workspace_bytes(specs, False), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(cca.grouped_workspace_bytes(specs, True), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the lanes outside the capture
        cca.fwd_grouped(specs, outs, ws_f)
        cca.bwd_grouped(specs, outs, dos, grads, ws_b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cca.fwd_grouped(specs, outs, ws_f)
        cca.bwd_grouped(specs, outs, dos, grads, ws_b)
    for rep in range(3):
        for o, l in outs:
            o.zero_()
        for g in grads:
            for t in g:
                t.fill_(1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (o, l), (eo, el) in zip(outs, eager_o):
            assert torch.equal(o, eo), rep
            if l is not None:
                assert torch.equal(l, el), rep
        for g, eg in zip(grads, eager_g):
            for a, b in zip(g, eg):
                assert torch.equal(a, b), rep


def test_grouped_with_an_empty_group(gdpa_lib):
    # A group whose samples are all empty runs nothing and leaves the others intact.
    cca = gdpa_lib
    a = gi.make_gdpa_inputs(gi.small_config(gi.EVENT_TYPES["conversion"], batch=3, lengths=("explicit", [40, 0, 77])),
                            seed=35, sharp=True)
    e = gi.make_gdpa_inputs(gi.small_config(gi.EVENT_TYPES["impression"], batch=2, lengths=("explicit", [0, 0])),
                            seed=36)
    specs = [cca.GroupSpec(x.q.cuda(), x.offsets.cuda(), x.k.cuda(), x.v.cuda(), phi=phi)
             for x, phi in ((a, "softmax"), (e, "silu"), (a, "silu"))]
    dos = [x.do.cuda() for x in (a, e, a)]
    outs = cca.fwd_grouped(specs)
    grads = cca.bwd_grouped(specs, outs, dos)
    torch.cuda.synchronize()
    assert outs[1][0].numel() == 0
    assert torch.count_nonzero(grads[1][1]) == 0 or grads[1][1].numel() == 0   # empty samples: dK = 0
    for i, phi in ((0, "softmax"), (2, "silu")):
        o_r, _ = orc.gdpa_forward(a.q, a.offsets, a.k, a.v, phi)
        dq_r, dk_r, dv_r = orc.gdpa_backward(a.q, a.offsets, a.k, a.v, a.do, phi)
        for got, ref in ((outs[i][0], o_r), (grads[i][0], dq_r), (grads[i][1], dk_r), (grads[i][2], dv_r)):
            assert max_abs_rel(got, ref) <= TOL["bf16"]
