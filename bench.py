#!/usr/bin/env python3
"""GDPA benchmark on one MI355X.

Default workload: the stacked jagged workload - 4 residual GDPA layers with
generated K/V, forward and backward, B=1024 samples with log-normal lengths
(median 1024, max 8192, T = 1,438,675 tokens at seed 0), H=8, d=128, n_kv=256,
context width 512, phi = SiLU (--phi selects another elementwise map).  One step
runs every stage of the path: weight generation (K, V = C W), GDPA forward with
the residual add, GDPA backward with dK/dV reduced per sample and dX = dX' + dQ,
and the weight gradients C^T dK, C^T dV.

`value` is GDPA forward+backward TFLOP/s over the whole step (algorithmic
FLOPs 12*T*H*n*d per layer, the weight-generation time counted in the
denominator, its FLOPs not in the numerator).  `gdpa_only_tflops` divides the
same FLOPs by the GDPA kernels' own time.  Prints one JSON line.

`roofline` describes the kernel with the largest share of the step: achieved
algorithmic bytes (or FLOPs) per launch over its average launch time, timed
with HIP events on the stream the library launches on.  `roofline.traffic` is
the HBM traffic per launch measured by rocprofv3 counters (FETCH_SIZE and
WRITE_SIZE, each scaled by the same counter's reading for a plain device copy
of known size, see --calibrate-copy); it is read from the committed summary in
profiles/ and reported only while the kernel sources still hash to the value
recorded there.

    python bench.py [--steps K] [--warmup W] [--config {2,3,4,5}] [--phi softmax|silu|relu|gelu|identity]
    python bench.py --calibrate-copy MIB   # plain copy of MIB MiB, for counter scaling
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0
METRIC = "GDPA fwd / fwd+bwd TFLOP/s and % of bf16 MFMA peak, jagged batch, 1 MI355X"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5, choices=[2, 3, 4, 5])
    ap.add_argument("--phi", default=None, choices=[None, "softmax", "silu", "relu", "gelu", "identity"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stats-steps", type=int, default=0,
                    help="steps of the statistics pass (default: >= 50 and >= 1 s); small values for profiler runs")
    ap.add_argument("--op", default="gdpa", choices=["gdpa", "swa", "pma", "jagged_kv", "layers", "biased",
                                                   "grouped"],
                    help="swa: sliding-window self-attention on the stacked workload's batch; "
                         "pma: seed pooling attention over that batch; jagged_kv: GDPA fwd+bwd with "
                         "per-sample context row counts (the fwd+bwd workload's batch); layers: the "
                         "Kunlun layer stack (GDPA + pooling + self-attention) on the stacked workload; "
                         "biased: GDPA fwd+bwd with FFN biases on the fwd+bwd workload; grouped: one "
                         "grouped call over the event types' GDPA problems")
    ap.add_argument("--schedule", default="compskip", choices=["compskip", "full"],
                    help="layer schedule of --op layers (the other one is timed alongside)")
    ap.add_argument("--window", type=int, default=512, help="window of --op swa")
    ap.add_argument("--seeds", type=int, default=32, help="seeds of --op pma (1..32)")
    ap.add_argument("--record-traffic", nargs=2, default=None, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="rewrite the committed traffic record of --config/--phi (or --op pma) from "
                         "two rocprofv3 counter runs of this script (FETCH_SIZE, then WRITE_SIZE; "
                         "their -d output folders), keeping the record's kernel lists and its copy "
                         "calibration; no GPU is used")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB three times (counter calibration)")
    return ap.parse_args()


CSRC = os.path.join(ROOT, "context_cross_attention_amd", "csrc")
# Committed counter records of HBM traffic, one per bench workload ((config, phi) or op).
TRAFFIC_FILES = {
    (5, "silu"): "traffic_stacked_b1024_h8_d128_n256_silu.json",
    (3, "softmax"): "traffic_fwd_b512_h8_d128_n512_softmax.json",
    (4, "softmax"): "traffic_fwdbwd_b256_h4_d128_n1024_softmax.json",
    "pma": "traffic_pma_b1024_h8_d128_m32.json",
}
# Shared device and launch headers: part of every call's kernels.
COMMON_SOURCES = ("gdpa_device.h", "gdpa_launch.h")


def traffic_file(key):
    """Path of the counter record of workload `key`, or None when none was taken."""
    name = TRAFFIC_FILES.get(key)
    return os.path.join(ROOT, "profiles", name) if name else None


def source_hash(sources):
    """sha256 over the named kernel sources and the shared headers, to tie a counter
    reading to the kernel version it was taken on."""
    h = hashlib.sha256()
    for name in sorted(set(sources) | set(COMMON_SOURCES)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(stage, path):
    """HBM bytes per launch of `stage` from a committed counter record, or None (no
    record for the workload, no reading for the stage, or the sources the record names
    changed since it was taken)."""
    if path is None:
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(stage)
    if not k or not k.get("sources") or k.get("source_sha256") != source_hash(k["sources"]):
        return None
    return k.get("bytes_per_launch")


def _counter_means(folder, counter):
    """Mean value of `counter` per dispatch, by kernel name (template arguments kept,
    namespace and parameter list dropped), over every rocprofv3 counter CSV under
    `folder`."""
    import csv
    import glob
    per = {}
    for path in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                name = row["Kernel_Name"]
                name = name[len("void "):] if name.startswith("void ") else name
                name = name.split("(")[0].replace("gdpa::", "")
                key = (name, row["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    sums = {}
    for (name, _), v in per.items():
        t = sums.setdefault(name, [0.0, 0])
        t[0] += v
        t[1] += 1
    return {name: tot / cnt for name, (tot, cnt) in sums.items()}


def record_traffic(args):
    """`--record-traffic`: rewrite the committed record of the workload that --config /
    --phi (or --op pma) name."""
    import gdpa_inputs as gi
    key = "pma" if args.op == "pma" else (args.config, args.phi or gi.CONFIGS[args.config].phis[0])
    path = traffic_file(key)
    if path is None:
        sys.exit(f"no traffic record for workload {key}")
    rewrite_traffic_record(path, args.record_traffic[0], args.record_traffic[1], " ".join(sys.argv[1:]))


def rewrite_traffic_record(path, fetch_dir, write_dir, cmdline):
    """Rewrite the traffic record at `path` (JSON and its Markdown summary) from the
    FETCH_SIZE and WRITE_SIZE counter runs in `fetch_dir` and `write_dir`: per stage,
    the per-dispatch means of its kernels are summed (one launch of the stage runs each
    once), scaled by the record's copy calibration, and tied to the current sources by
    their hash.  `cmdline` is the bench.py argument list quoted in the summary."""
    with open(path) as f:
        rec = json.load(f)
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    cal = rec["calibration"]
    rows = []
    for stage, k in rec["kernels"].items():
        missing = [n for n in k["kernels"] if n not in fetch or n not in write]
        if missing:
            sys.exit(f"{stage}: no counter readings for {missing}")
        k["fetch_kib"] = round(sum(fetch[n] for n in k["kernels"]), 1)
        k["write_kib"] = round(sum(write[n] for n in k["kernels"]), 1)
        k["bytes_per_launch"] = int(round((k["fetch_kib"] * cal["fetch_scale"] + k["write_kib"] * cal["write_scale"])
                                          * 1024))
        k["source_sha256"] = source_hash(k["sources"])
        rows.append((stage, k))
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    md = os.path.splitext(path)[0] + ".md"
    lines = [f"# HBM traffic per launch: {rec['workload']}", "",
             "Counters `FETCH_SIZE` and `WRITE_SIZE` (KiB per dispatch), each in its own rocprofv3",
             "run, run from /tmp with TMPDIR=/tmp, repo at $R; the record is then rewritten from",
             "the two output folders:", "", "```"]
    lines += [rec["commands"][c] for c in ("bench_fetch", "bench_write")]
    lines += [f"python3 $R/bench.py {cmdline}"]
    lines += [rec["commands"][c] for c in ("copy_fetch", "copy_write")]
    lines += ["```", "",
              f"Calibration (the copy runs above): a plain device copy of {cal['copy_bytes'] >> 20} MiB reads "
              f"`FETCH_SIZE` = {cal['fetch_kib']} KiB and", f"`WRITE_SIZE` = {cal['write_kib']} KiB, so fetched "
              f"bytes = {cal['fetch_scale']:.4f} x FETCH_SIZE x 1024 and written", f"bytes = "
              f"{cal['write_scale']:.4f} x WRITE_SIZE x 1024.", "",
              "| call | kernels | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes / launch (scaled) | "
              "algorithmic bytes / launch | ratio |", "|---|---|---|---|---|---|---|"]
    for stage, k in rows:
        alg = k.get("algorithmic_bytes_per_launch")
        lines.append(f"| {stage} | {', '.join('`' + n + '`' for n in k['kernels'])} | {k['fetch_kib']} | "
                     f"{k['write_kib']} | {k['bytes_per_launch'] / 1e9:.3f} GB | "
                     + (f"{alg / 1e9:.3f} GB | {k['bytes_per_launch'] / alg:.2f} |" if alg else "- | - |"))
    lines += ["", f"The machine-readable record is `{os.path.basename(path)}`; each entry carries the sha256 "
              "of the sources its kernels are built from (with the shared device and launch headers), and "
              "`bench.py` reports `roofline.traffic` for this workload from it only while they still match.", ""]
    with open(md, "w") as f:
        f.write("\n".join(lines))
    print(json.dumps({"record": os.path.relpath(path, ROOT),
                      "bytes_per_launch": {st: k["bytes_per_launch"] for st, k in rows}}))


def calibrate_copy(mib):
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))


# ---------------------------------------------------------------------------
# algorithmic work per launch
# ---------------------------------------------------------------------------

def gdpa_units(kind, T, B, H, d, n, phi, residual=False):
    """(FLOPs, HBM bytes) per launch: each tensor moved once, bf16 data, fp32 lse/dvec."""
    tok = T * H * d * 2
    kv = B * n * H * d * 2
    if kind == "gdpa_fwd":
        flops = 4.0 * T * H * n * d
        # the residual of a stacked layer is the query tensor itself: counted once
        byts = 2 * tok + 2 * kv + (T * H * 4 if phi == "softmax" else 0)
    else:
        flops = 8.0 * T * H * n * d
        byts = 3 * tok + 4 * kv
        if phi == "softmax":
            byts += tok + 2 * T * H * 4  # O for rowsum(dO*O), lse, dvec round trip
    return flops, byts


def gemm_units(M, N, K):
    return 2.0 * M * N * K, 2.0 * (M * K + K * N + M * N)


class Marks:
    """HIP events around library calls on the current stream, per category."""

    def __init__(self, torch):
        self.torch = torch
        self.open = {}
        self.pairs = {}
        self.enabled = False

    def __call__(self, name, start):
        if not self.enabled:
            return
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record()
        if start:
            self.open[name] = ev
        else:
            self.pairs.setdefault(name, []).append((self.open.pop(name), ev))

    def totals_ms(self):
        return {k: sum(a.elapsed_time(b) for a, b in v) for k, v in self.pairs.items()}

    def counts(self):
        return {k: len(v) for k, v in self.pairs.items()}


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample of the same inputs
# ---------------------------------------------------------------------------

def blas_threads():
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        n = [i["num_threads"] for i in info if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count() or 1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class CpuClock:
    """Wall time and this process's CPU time (all its threads, user + system) over a
    region: their ratio is the number of cores the region kept busy on average."""

    def __enter__(self):
        import resource
        self._r = resource
        u = resource.getrusage(resource.RUSAGE_SELF)
        self.cpu0, self.t0 = u.ru_utime + u.ru_stime, time.perf_counter()
        return self

    def __exit__(self, *exc):
        u = self._r.getrusage(self._r.RUSAGE_SELF)
        self.wall = time.perf_counter() - self.t0
        self.cpu = u.ru_utime + u.ru_stime - self.cpu0
        return False

    def fields(self):
        eff = self.cpu / self.wall if self.wall > 0 else 0.0
        return {"cores": max(1, int(round(eff))), "cores_effective": round(eff, 2),
                "threads_available": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
                else (os.cpu_count() or 1),
                "blas_threads": blas_threads(), "cpu_model": cpu_model(), "processes": 1}


def pick_samples(lengths, per_token_flops, budget_flops, cap):
    chosen, acc = [], 0.0
    for b, L in enumerate(lengths):
        if L == 0:
            continue
        chosen.append(b)
        acc += L * per_token_flops
        if acc >= budget_flops or len(chosen) >= cap:
            break
    return chosen


def cpu_baseline_stacked(inp, cfg, phi):
    import numpy as np
    from oracle import gdpa_oracle as orc
    per_tok = 12.0 * cfg.layers * cfg.heads * cfg.n_kv * cfg.head_dim
    samples = pick_samples(inp.lengths, per_tok, 3.0e11, 16)
    off = inp.offsets.numpy().astype(np.int64)
    rows = np.concatenate([np.arange(off[b], off[b + 1]) for b in samples])
    sub_off = np.concatenate([[0], np.cumsum([inp.lengths[b] for b in samples])])
    x0 = inp.x0[rows]
    g = inp.do[rows]
    ctx = inp.ctx[samples]
    with CpuClock() as clk:
        xs = orc.stacked_forward(x0, sub_off, ctx, inp.w_k, inp.w_v, cfg.heads, cfg.n_kv, phi)
        orc.stacked_backward(xs, sub_off, ctx, inp.w_k, inp.w_v, g, cfg.heads, cfg.n_kv, phi)
    dt = clk.wall
    tokens = int(sub_off[-1])
    flops = per_tok * tokens
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", **clk.fields(), "kind": "oracle",
            "sample": f"stacked {cfg.layers}-layer {phi} fwd+bwd incl. weight generation on samples "
                      f"{samples[0]}..{samples[-1]} ({len(samples)} of {cfg.batch}, {tokens} tokens); "
                      f"GDPA FLOPs {flops / 1e9:.1f} G in {dt:.1f} s (numpy float64, one process; "
                      f"BLAS products multithreaded, elementwise work on one thread)",
            "seconds": round(dt, 2)}


def cpu_baseline_single(inp, cfg, phi):
    import numpy as np
    from oracle import gdpa_oracle as orc
    per_tok = (12.0 if cfg.backward else 4.0) * cfg.heads * cfg.n_kv * cfg.head_dim
    samples = pick_samples(inp.lengths, per_tok, 2.5e11, cfg.batch)
    with CpuClock() as clk:
        orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, phi, samples=samples)
        if cfg.backward:
            orc.gdpa_backward(inp.q, inp.offsets, inp.k, inp.v, inp.do, phi, samples=samples)
    dt = clk.wall
    tokens = int(sum(inp.lengths[b] for b in samples))
    flops = per_tok * tokens
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", **clk.fields(), "kind": "oracle",
            "sample": f"{'fwd+bwd' if cfg.backward else 'fwd'} {phi} on {len(samples)} of {cfg.batch} "
                      f"samples ({tokens} tokens); {flops / 1e9:.1f} GFLOP in {dt:.1f} s (numpy float64, "
                      f"one process)",
            "seconds": round(dt, 2)}


# ---------------------------------------------------------------------------
# sliding-window self-attention (--op swa)
# ---------------------------------------------------------------------------

def swa_pairs(lengths, w):
    """Number of (token, key) pairs in the windows: sum over samples and positions of min(i + 1, w)."""
    tot = 0
    for L in lengths:
        L = int(L)
        m = min(L, w)
        tot += m * (m + 1) // 2 + (L - m) * w
    return tot


def run_swa(args):
    import numpy as np
    import torch

    import context_cross_attention_amd as cca
    import gdpa_inputs as gi

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cca.load()
    cfg = gi.CONFIGS[5]
    w = args.window
    H, d, B = cfg.heads, cfg.head_dim, cfg.batch
    inp = gi.make_swa_inputs(cfg.lengths, B, H, d, seed=args.seed)
    T = inp.total_tokens
    q, k, v, do = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.do))
    off = inp.offsets.cuda()
    o = torch.empty_like(q)
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(cca.swa_workspace_bytes(q, off, w, True), dtype=torch.uint8, device="cuda")
    marks = Marks(torch)

    def step():
        marks("swa_fwd", True)
        cca.swa_fwd(q, off, k, v, w, out=o, lse=lse, workspace=ws)
        marks("swa_fwd", False)
        marks("swa_bwd", True)
        cca.swa_bwd(q, off, k, v, o, lse, do, w, dq=dq, dk=dk, dv=dv, workspace=ws)
        marks("swa_bwd", False)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    marks.enabled = True
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    marks.enabled = False
    pairs = swa_pairs(inp.lengths, w)
    f_fwd, f_bwd = 4.0 * d * H * pairs, 8.0 * d * H * pairs
    tok = T * H * d * 2
    units = {"swa_fwd": (f_fwd, 4 * tok + 4 * T * H), "swa_bwd": (f_bwd, 8 * tok + 8 * T * H)}
    totals, counts = marks.totals_ms(), marks.counts()
    dom = max(totals, key=lambda x: totals[x])
    t_dom = totals[dom] / counts[dom] * 1e-3
    f_dom, b_dom = units[dom]
    if b_dom / (PEAK_HBM_GBS * 1e9) >= f_dom / (PEAK_BF16_TFLOPS * 1e12):
        roof = {"bound": "hbm", "achieved": round(b_dom / t_dom / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(f_dom / t_dom / 1e12, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    roof.update(frac=round(roof["achieved"] / roof["peak"], 4), traffic=None, kernel=dom,
                launch_ms=round(totals[dom] / counts[dom], 4),
                algorithmic_per_launch={"flops": f_dom, "bytes": b_dom})
    value = (f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": "sliding-window self-attention fwd+bwd TFLOP/s, jagged batch, 1 MI355X",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded numpy draws as in gdpa_inputs.make_swa_inputs)",
        "config": {"workload": f"sliding-window self-attention fwd+bwd, window {w}: B={B} samples, lengths "
                               f"log-normal (median {cfg.lengths[1]}, max {cfg.lengths[2]}), T={T}, H={H}, d={d}",
                   "window": w, "tokens": T, "heads": H, "head_dim": d, "pairs": pairs, "seed": args.seed},
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "breakdown_ms_per_step": {x: round(totals[x] / args.steps, 4) for x in totals},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from oracle import swa_oracle as swo
        chosen, cost = [], 0.0
        for b in range(B):
            if inp.lengths[b] == 0:
                continue
            chosen.append(b)
            cost += 12.0 * float(inp.lengths[b]) ** 2 * H * d   # the oracle forms whole L x L products
            if cost >= 3.0e11:
                break
        clk = CpuClock().__enter__()
        swo.swa_forward(inp.q, inp.offsets, inp.k, inp.v, w, samples=chosen)
        swo.swa_backward(inp.q, inp.offsets, inp.k, inp.v, inp.do, w, samples=chosen)
        clk.__exit__(None, None, None)
        dt = clk.wall
        p_s = swa_pairs([inp.lengths[b] for b in chosen], w)
        fl = 12.0 * d * H * p_s
        out["cpu_baseline"] = {"value": fl / dt / 1e12, "unit": "TFLOP/s", **clk.fields(),
                               "kind": "oracle",
                               "sample": f"fwd+bwd on samples {chosen[0]}..{chosen[-1]} ({len(chosen)} of {B}); "
                                         f"{fl / 1e9:.1f} GFLOP of window pairs in {dt:.1f} s (numpy float64, "
                                         f"dense L x L per sample)", "seconds": round(dt, 2)}
    print(json.dumps(out))


# ---------------------------------------------------------------------------
# GDPA with a jagged context (--op jagged_kv)
# ---------------------------------------------------------------------------

JAGGED_KV_COUNTS = ("uniform", 64, 1024)


def run_jagged_kv(args):
    import numpy as np
    import torch

    import context_cross_attention_amd as cca
    import gdpa_inputs as gi

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cca.load()
    cfg = gi.CONFIGS[4]
    phi = args.phi or "softmax"
    H, d, B = cfg.heads, cfg.head_dim, cfg.batch
    inp = gi.make_jagged_kv_inputs(cfg.lengths, JAGGED_KV_COUNTS, B, H, d, seed=args.seed)
    T, n_max = int(inp.offsets[-1]), inp.n_kv
    q, k, v, do = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.do))
    off, ko = inp.offsets.cuda(), inp.kv_offsets.cuda()
    o = torch.empty_like(q)
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(cca.jagged_kv_workspace_bytes(q, off, k, n_max, phi, True), 1),
                     dtype=torch.uint8, device="cuda")
    marks = Marks(torch)

    def step():
        marks("gdpa_fwd", True)
        cca.fwd_jagged_kv(q, off, ko, k, v, n_max, phi=phi, out=o, lse=lse, workspace=ws)
        marks("gdpa_fwd", False)
        marks("gdpa_bwd", True)
        cca.bwd_jagged_kv(q, off, ko, k, v, n_max, o, lse, do, phi=phi, dq=dq, dk=dk, dv=dv, workspace=ws)
        marks("gdpa_bwd", False)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    marks.enabled = True
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    marks.enabled = False
    pairs = float(np.dot(inp.lengths, inp.kv_counts))  # (token, context row) pairs
    rows = int(inp.kv_counts.sum())
    tok, kvb = T * H * d * 2, rows * H * d * 2
    f_fwd, f_bwd = 4.0 * d * H * pairs, 8.0 * d * H * pairs
    b_fwd = 2 * tok + 2 * kvb + (T * H * 4 if phi == "softmax" else 0)
    b_bwd = 3 * tok + 4 * kvb + ((tok + 2 * T * H * 4) if phi == "softmax" else 0)
    units = {"gdpa_fwd": (f_fwd, b_fwd), "gdpa_bwd": (f_bwd, b_bwd)}
    totals, counts = marks.totals_ms(), marks.counts()
    dom = max(totals, key=lambda x: totals[x])
    t_dom = totals[dom] / counts[dom] * 1e-3
    f_dom, b_dom = units[dom]
    if b_dom / (PEAK_HBM_GBS * 1e9) >= f_dom / (PEAK_BF16_TFLOPS * 1e12):
        roof = {"bound": "hbm", "achieved": round(b_dom / t_dom / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(f_dom / t_dom / 1e12, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    roof.update(frac=round(roof["achieved"] / roof["peak"], 4), traffic=None, kernel=dom,
                launch_ms=round(totals[dom] / counts[dom], 4),
                algorithmic_per_launch={"flops": f_dom, "bytes": b_dom})
    value = (f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": "GDPA fwd+bwd TFLOP/s with a jagged context, jagged batch, 1 MI355X",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded numpy draws as in gdpa_inputs.make_jagged_kv_inputs)",
        "config": {"workload": f"GDPA fwd+bwd, phi={phi}, jagged context: B={B}, L~U[256,2048], context rows "
                               f"~U[{JAGGED_KV_COUNTS[1]},{JAGGED_KV_COUNTS[2]}] per sample (max {n_max}), "
                               f"T={T}, H={H}, d={d}",
                   "tokens": T, "context_rows": rows, "heads": H, "head_dim": d, "phi": phi, "seed": args.seed},
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "breakdown_ms_per_step": {x: round(totals[x] / args.steps, 4) for x in totals},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from oracle import gdpa_oracle as orc
        chosen, cost = [], 0.0
        for b in range(B):
            chosen.append(b)
            cost += 12.0 * float(inp.lengths[b]) * float(inp.kv_counts[b]) * H * d
            if cost >= 1.3e12:
                break
        clk = CpuClock().__enter__()
        orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, phi, samples=chosen, kv_offsets=inp.kv_offsets)
        orc.gdpa_backward(inp.q, inp.offsets, inp.k, inp.v, inp.do, phi, samples=chosen, kv_offsets=inp.kv_offsets)
        clk.__exit__(None, None, None)
        dt = clk.wall
        out["cpu_baseline"] = {"value": cost / dt / 1e12, "unit": "TFLOP/s", **clk.fields(),
                               "kind": "oracle",
                               "sample": f"fwd+bwd on samples 0..{chosen[-1]} ({len(chosen)} of {B}); "
                                         f"{cost / 1e9:.1f} GFLOP in {dt:.1f} s (numpy float64)",
                               "seconds": round(dt, 2)}
    print(json.dumps(out))


# ---------------------------------------------------------------------------
# GDPA with FFN biases (--op biased)
# ---------------------------------------------------------------------------


def run_biased(args):
    import torch

    import context_cross_attention_amd as cca
    import gdpa_inputs as gi

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cca.load()
    cfg = gi.CONFIGS[4]
    phi = args.phi or "silu"
    H, d, n, B = cfg.heads, cfg.head_dim, cfg.n_kv, cfg.batch
    inp = gi.make_gdpa_inputs(cfg, seed=args.seed)
    T = inp.total_tokens
    sb_h, ob_h = gi.draw_ffn_biases(args.seed + 1, (B, n, H), B, H, d)
    q, off, k, v, do = (t.cuda() for t in (inp.q, inp.offsets, inp.k, inp.v, inp.do))
    sb, ob = sb_h.cuda(), ob_h.cuda()
    o = torch.empty_like(q)
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dsb, dob = torch.empty_like(sb), torch.empty_like(ob)
    ws = torch.empty(max(cca.biased_workspace_bytes(q, off, k, phi, True, True), 1 << 20), dtype=torch.uint8,
                     device="cuda")
    marks = Marks(torch)

    def step_biased():
        marks("gdpa_fwd_biased", True)
        cca.fwd_biased(q, off, k, v, sb, ob, phi=phi, out=o, lse=lse, workspace=ws)
        marks("gdpa_fwd_biased", False)
        marks("gdpa_bwd_biased", True)
        cca.bwd_biased(q, off, k, v, sb, ob, o, lse, do, phi=phi, workspace=ws, dq=dq, dk=dk, dv=dv,
                       d_score_bias=dsb, d_out_bias=dob)
        marks("gdpa_bwd_biased", False)

    def step_plain():
        cca.fwd(q, off, k, v, phi=phi, out=o, lse=lse, workspace=ws)
        cca.bwd(q, off, k, v, o, lse, do, phi=phi, dq=dq, dk=dk, dv=dv, workspace=ws)

    def timed(step, use_marks):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        marks.enabled = use_marks
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        marks.enabled = False
        return (time.perf_counter() - t0) * 1e3 / args.steps

    ms_plain = timed(step_plain, False)
    ms_per_step = timed(step_biased, True)
    pairs = float(inp.lengths.sum()) * n
    tok, kvb, sbb = T * H * d * 2, B * n * H * d * 2, B * n * H * 4
    f_fwd, f_bwd = 4.0 * d * H * pairs, 8.0 * d * H * pairs
    extra_fwd = 4.0 * d * H * pairs if phi == "softmax" else 0.0  # P V recomputed in the backward
    b_fwd = 2 * tok + 2 * kvb + sbb + (T * H * 4 if phi == "softmax" else 0)
    b_bwd = 3 * tok + 4 * kvb + 2 * sbb + tok + ((2 * T * H * 4) if phi == "softmax" else 0)
    units = {"gdpa_fwd_biased": (f_fwd, b_fwd), "gdpa_bwd_biased": (f_bwd + extra_fwd, b_bwd)}
    totals, counts = marks.totals_ms(), marks.counts()
    dom = max(totals, key=lambda x: totals[x])
    t_dom = totals[dom] / counts[dom] * 1e-3
    f_dom, b_dom = units[dom]
    roof = {"bound": "mfma", "achieved": round(f_dom / t_dom / 1e12, 1), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s"}
    roof.update(frac=round(roof["achieved"] / roof["peak"], 4), traffic=None, kernel=dom,
                launch_ms=round(totals[dom] / counts[dom], 4),
                algorithmic_per_launch={"flops": f_dom, "bytes": b_dom})
    value = (f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": "GDPA fwd+bwd TFLOP/s with FFN biases, jagged batch, 1 MI355X",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded numpy draws as in gdpa_inputs.make_gdpa_inputs and draw_ffn_biases)",
        "config": {"workload": f"GDPA fwd+bwd with a score bias per context row and an output bias, phi={phi}: "
                               f"B={B}, L~U[256,2048], T={T}, H={H}, d={d}, n={n}",
                   "tokens": T, "heads": H, "head_dim": d, "n_kv": n, "phi": phi, "seed": args.seed},
        "unbiased_ms_per_step": round(ms_plain, 4),
        "bias_overhead": round(ms_per_step / ms_plain - 1.0, 4),
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "breakdown_ms_per_step": {x: round(totals[x] / args.steps, 4) for x in totals},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from oracle import gdpa_oracle as orc
        chosen, cost = [], 0.0
        for b in range(B):
            chosen.append(b)
            cost += 12.0 * float(inp.lengths[b]) * n * H * d
            if cost >= 4.5e11:
                break
        clk = CpuClock().__enter__()
        orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, phi, samples=chosen, score_bias=sb_h, out_bias=ob_h)
        orc.gdpa_backward(inp.q, inp.offsets, inp.k, inp.v, inp.do, phi, samples=chosen, score_bias=sb_h,
                          bias_grads=True)
        clk.__exit__(None, None, None)
        dt = clk.wall
        out["cpu_baseline"] = {"value": cost / dt / 1e12, "unit": "TFLOP/s", **clk.fields(),
                               "kind": "oracle",
                               "sample": f"fwd+bwd on samples 0..{chosen[-1]} ({len(chosen)} of {B}); "
                                         f"{cost / 1e9:.1f} GFLOP in {dt:.1f} s (numpy float64)",
                               "seconds": round(dt, 2)}
    print(json.dumps(out))


# ---------------------------------------------------------------------------
# grouped launch over the event types (--op grouped)
# ---------------------------------------------------------------------------


def run_grouped(args):
    import torch

    import context_cross_attention_amd as cca
    import gdpa_inputs as gi

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cca.load()
    phi = args.phi or "silu"
    events = gi.make_event_inputs(seed=args.seed)
    specs, dos = [], []
    for inp in events.values():
        specs.append(cca.GroupSpec(inp.q.cuda(), inp.offsets.cuda(), inp.k.cuda(), inp.v.cuda(), phi=phi))
        dos.append(inp.do.cuda())
    outs = [(torch.empty_like(sp.q), torch.empty((sp.q.shape[0], sp.q.shape[1]), dtype=torch.float32,
                                                 device="cuda")) for sp in specs]
    grads = [(torch.empty_like(sp.q), torch.empty_like(sp.k), torch.empty_like(sp.v)) for sp in specs]
    ws_f = torch.empty(cca.grouped_workspace_bytes(specs, False), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(cca.grouped_workspace_bytes(specs, True), dtype=torch.uint8, device="cuda")
    ws_1 = torch.empty(max(max(cca.workspace_bytes(cca.make_problem(sp.q, sp.offsets, sp.k, phi, None), bw)
                               for sp in specs for bw in (False, True)), 1), dtype=torch.uint8, device="cuda")
    marks = Marks(torch)

    def step_grouped():
        marks("gdpa_fwd_grouped", True)
        cca.fwd_grouped(specs, outs, ws_f)
        marks("gdpa_fwd_grouped", False)
        marks("gdpa_bwd_grouped", True)
        cca.bwd_grouped(specs, outs, dos, grads, ws_b)
        marks("gdpa_bwd_grouped", False)

    def step_serial():
        for i, sp in enumerate(specs):
            o, lse = outs[i]
            cca.fwd(sp.q, sp.offsets, sp.k, sp.v, phi=phi, out=o, lse=lse, workspace=ws_1)
            cca.bwd(sp.q, sp.offsets, sp.k, sp.v, o, lse, dos[i], phi=phi, dq=grads[i][0], dk=grads[i][1],
                    dv=grads[i][2], workspace=ws_1)

    def timed(step, use_marks):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        marks.enabled = use_marks
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        marks.enabled = False
        return (time.perf_counter() - t0) * 1e3 / args.steps

    ms_serial = timed(step_serial, False)
    ms_per_step = timed(step_grouped, True)
    f_fwd = f_bwd = 0.0
    per_event = {}
    for name, inp in events.items():
        cfg = inp.cfg
        pairs = float(inp.lengths.sum()) * cfg.n_kv
        f = 4.0 * cfg.heads * cfg.head_dim * pairs
        f_fwd += f
        f_bwd += 2 * f
        per_event[name] = {"tokens": int(inp.lengths.sum()), "heads": cfg.heads, "head_dim": cfg.head_dim,
                           "n_kv": cfg.n_kv, "gflop_fwd_bwd": round(3 * f / 1e9, 1)}
    totals, counts = marks.totals_ms(), marks.counts()
    units = {"gdpa_fwd_grouped": f_fwd, "gdpa_bwd_grouped": f_bwd}
    dom = max(totals, key=lambda x: totals[x])
    t_dom = totals[dom] / counts[dom] * 1e-3
    roof = {"bound": "mfma", "achieved": round(units[dom] / t_dom / 1e12, 1), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s"}
    roof.update(frac=round(roof["achieved"] / roof["peak"], 4), traffic=None, kernel=dom,
                launch_ms=round(totals[dom] / counts[dom], 4), algorithmic_per_launch={"flops": units[dom]},
                note="one call of several kernels on up to four streams; the time is the call's span")
    value = (f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": "GDPA fwd+bwd TFLOP/s over several event types in one grouped call, 1 MI355X",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded numpy draws as in gdpa_inputs.make_event_inputs)",
        "config": {"workload": "GDPA fwd+bwd, phi=" + phi + ", one problem per event type: "
                               + "; ".join(cfg.name for cfg in gi.EVENT_TYPES.values()),
                   "events": per_event, "phi": phi, "seed": args.seed},
        "serial_ms_per_step": round(ms_serial, 4),
        "grouped_speedup": round(ms_serial / ms_per_step, 4),
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "breakdown_ms_per_step": {x: round(totals[x] / args.steps, 4) for x in totals},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from oracle import gdpa_oracle as orc
        inp = events["click"]
        cfg = inp.cfg
        chosen, cost = [], 0.0
        for b in range(cfg.batch):
            chosen.append(b)
            cost += 12.0 * float(inp.lengths[b]) * cfg.n_kv * cfg.heads * cfg.head_dim
            if cost >= 3.5e11:
                break
        clk = CpuClock().__enter__()
        orc.gdpa_forward(inp.q, inp.offsets, inp.k, inp.v, phi, samples=chosen)
        orc.gdpa_backward(inp.q, inp.offsets, inp.k, inp.v, inp.do, phi, samples=chosen)
        clk.__exit__(None, None, None)
        dt = clk.wall
        out["cpu_baseline"] = {"value": cost / dt / 1e12, "unit": "TFLOP/s", **clk.fields(),
                               "kind": "oracle",
                               "sample": f"fwd+bwd of the click events on samples 0..{chosen[-1]} "
                                         f"({len(chosen)} of {cfg.batch}); {cost / 1e9:.1f} GFLOP in {dt:.1f} s "
                                         f"(numpy float64)",
                               "seconds": round(dt, 2)}
    print(json.dumps(out))


# ---------------------------------------------------------------------------
# the Kunlun layer stack with the CompSkip schedule (--op layers)
# ---------------------------------------------------------------------------

def run_layers(args):
    import torch

    import context_cross_attention_amd as cca
    import gdpa_inputs as gi
    from context_cross_attention_amd.layers import KunlunLayers

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cca.load()
    cfg = gi.CONFIGS[5]
    m, w = args.seeds, args.window
    H, d, B, n, c, L = cfg.heads, cfg.head_dim, cfg.batch, cfg.n_kv, cfg.ctx_dim, cfg.layers
    inp = gi.make_layer_stack_inputs(cfg.lengths, B, H, d, n, c, layers=L, m=m, seed=args.seed)
    T = int(inp.offsets[-1])
    dev = "cuda"
    off, ctx = inp.offsets.to(dev), inp.ctx.to(dev)
    wk, wv, sd = ([t.to(dev) for t in ts] for ts in (inp.w_k, inp.w_v, inp.seeds))
    x0, dx = inp.x0.to(dev), inp.dx.to(dev)
    gz_all = [t.to(dev) for t in inp.dz]

    def time_schedule(schedule, marks):
        model = KunlunLayers(off, ctx, wk, wv, sd, H, n, T, w, schedule)
        gz = {l: gz_all[l] for l in range(L) if model.ops[l][1]}

        def step():
            model.forward(x0, mark=marks)
            model.backward(dx, gz, mark=marks)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        marks.enabled = True
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        marks.enabled = False
        del model
        torch.cuda.empty_cache()
        return ms

    other = "full" if args.schedule == "compskip" else "compskip"
    marks = Marks(torch)
    ms = time_schedule(args.schedule, marks)
    totals, counts = marks.totals_ms(), marks.counts()
    ms_other = time_schedule(other, Marks(torch))
    fl = layer_stack_flops(inp.lengths, H, d, n, c, m, w, L, args.schedule)
    fl_other = layer_stack_flops(inp.lengths, H, d, n, c, m, w, L, other)
    value = T / (ms * 1e-3)
    # Roofline of the largest stage per launch (the self-attention backward for the
    # default window), with the single-op models: SWA 8 d H FLOPs per pair and
    # 8 T H d bf16 + 8 T H bytes, plus the residual sum (4 reads, 1 write); GDPA as
    # gdpa_units.
    tok = T * H * d * 2
    per_launch = {"sa_bwd": (8.0 * d * H * swa_pairs(inp.lengths, w), 8 * tok + 8 * T * H + 5 * tok),
                  "gdpa_bwd": gdpa_units("gdpa_bwd", T, B, H, d, n, "silu", residual=True)}
    dom = max(totals, key=lambda x: totals[x])
    roof = None
    if dom in per_launch:
        t_dom = totals[dom] / counts[dom] * 1e-3
        f_dom, b_dom = per_launch[dom]
        if b_dom / (PEAK_HBM_GBS * 1e9) >= f_dom / (PEAK_BF16_TFLOPS * 1e12):
            roof = {"bound": "hbm", "achieved": round(b_dom / t_dom / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
        else:
            roof = {"bound": "mfma", "achieved": round(f_dom / t_dom / 1e12, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s"}
        roof.update(frac=round(roof["achieved"] / roof["peak"], 4), traffic=None, kernel=dom,
                    launch_ms=round(totals[dom] / counts[dom], 4),
                    algorithmic_per_launch={"flops": f_dom, "bytes": b_dom})
    out = {
        "metric": "Kunlun layer stack (GDPA + HSP pooling + self-attention) fwd+bwd tokens/s, jagged batch, 1 MI355X",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded numpy draws as in gdpa_inputs.make_layer_stack_inputs)",
        "config": {"workload": f"{L}-layer Kunlun stack, schedule {args.schedule}: B={B}, lengths log-normal "
                               f"(median {cfg.lengths[1]}, max {cfg.lengths[2]}), T={T}, H={H}, d={d}, n_kv={n}, "
                               f"ctx {c}, SiLU PFFN, {m} seeds, window {w}",
                   "schedule": args.schedule, "layers": L, "tokens": T, "seeds": m, "window": w, "seed": args.seed},
        "tflops": round(fl["total"] / (ms * 1e-3) / 1e12, 2),
        "flops_per_step": {k: round(v / 1e12, 3) for k, v in fl.items()},
        "breakdown_ms_per_step": {x: round(totals[x] / args.steps, 3) for x in totals},
        "compare": {"schedule": other, "ms_per_step": round(ms_other, 3),
                    "time_ratio": round(ms / ms_other, 4), "flop_ratio": round(fl["total"] / fl_other["total"], 4)},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from oracle import compskip_oracle as cso
        chosen, toks = [], 0
        for b in range(B):
            if 0 < inp.lengths[b] <= 1500:
                chosen.append(b)
                toks += int(inp.lengths[b])
            if toks >= 20000:
                break
        rows = torch.cat([torch.arange(int(inp.offsets[b]), int(inp.offsets[b + 1])) for b in chosen])
        sub_off = torch.zeros(len(chosen) + 1, dtype=torch.int64)
        sub_off[1:] = torch.cumsum(torch.as_tensor(inp.lengths[chosen]), 0)
        sub_ctx, sub_dz = inp.ctx[chosen], [z[chosen] for z in inp.dz]
        clk = CpuClock().__enter__()
        recs, _, zs = cso.forward(inp.x0[rows], sub_off, sub_ctx, inp.w_k, inp.w_v, inp.seeds, H, n, w,
                                  args.schedule)
        cso.backward(recs, sub_off, sub_ctx, inp.w_k, inp.w_v, inp.seeds, H, n, w, args.schedule, inp.dx[rows],
                     {l: sub_dz[l] for l in zs})
        clk.__exit__(None, None, None)
        dt = clk.wall
        out["cpu_baseline"] = {"value": round(toks / dt, 1), "unit": "tokens/s", **clk.fields(),
                               "kind": "oracle",
                               "sample": f"fwd+bwd of the {L}-layer stack on {len(chosen)} samples ({toks} tokens); "
                                         f"{dt:.1f} s (numpy float64)", "seconds": round(dt, 2)}
    print(json.dumps(out))


def layer_stack_flops(lengths, H, d, n, c, m, w, layers, schedule):
    """Algorithmic FLOPs of one forward + backward of the layer stack, per op kind:
    GDPA 12 T H n d; weight generation 4 GEMMs of 2 B (n H d) c; pooling 14 T H m d;
    self-attention 12 H d per in-window (token, key) pair."""
    T, B = float(sum(int(x) for x in lengths)), len(lengths)
    pairs = swa_pairs(lengths, w)
    out = {"gdpa": 0.0, "weightgen": 0.0, "hsp": 0.0, "sa": 0.0}
    for l in range(layers):
        full = schedule == "full"
        if full or l % 2 == 0:
            out["gdpa"] += 12.0 * T * H * n * d
            out["weightgen"] += 4 * 2.0 * B * (n * H * d) * c
            out["hsp"] += 14.0 * T * H * m * d
        if full or l % 2 == 1:
            out["sa"] += 12.0 * H * d * pairs
    out["total"] = sum(out.values())
    return out


# ---------------------------------------------------------------------------
# seed pooling attention (--op pma)
# ---------------------------------------------------------------------------

def pma_units(T, B, H, d, m):
    """(flops, algorithmic HBM bytes) of the forward and the backward calls."""
    tok = T * H * d * 2                       # one bf16 [T,H,d] tensor
    pooled = B * m * H * d * 2                # one bf16 [B,m,H,d] tensor
    small = m * H * d * 2 + B * m * H * 4     # seeds, LSE
    fwd = (4.0 * m * d * H * T, 2 * tok + pooled + small)
    bwd = (10.0 * m * d * H * T, 4 * tok + 2 * pooled + small + m * H * d * 2)
    return fwd, bwd


def run_pma(args):
    import torch

    import context_cross_attention_amd as cca
    import gdpa_inputs as gi

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cca.load()
    cfg = gi.CONFIGS[5]
    m = args.seeds
    H, d, B = cfg.heads, cfg.head_dim, cfg.batch
    inp = gi.make_pma_inputs(cfg.lengths, B, H, d, m, seed=args.seed)
    T = inp.total_tokens
    seeds, k, v, do = (t.cuda() for t in (inp.seeds, inp.k, inp.v, inp.do))
    off = inp.offsets.cuda()
    o = torch.empty((B, m, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, m, H), dtype=torch.float32, device="cuda")
    dseeds, dk, dv = torch.empty_like(seeds), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(cca.pma_workspace_bytes(seeds, off, k, True), dtype=torch.uint8, device="cuda")
    marks = Marks(torch)

    def step():
        marks("pma_fwd", True)
        cca.pma_fwd(seeds, off, k, v, out=o, lse=lse, workspace=ws)
        marks("pma_fwd", False)
        marks("pma_bwd", True)
        cca.pma_bwd(seeds, off, k, v, o, lse, do, d_seeds=dseeds, dk=dk, dv=dv, workspace=ws)
        marks("pma_bwd", False)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    marks.enabled = True
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    marks.enabled = False
    (f_fwd, b_fwd), (f_bwd, b_bwd) = pma_units(T, B, H, d, m)
    units = {"pma_fwd": (f_fwd, b_fwd), "pma_bwd": (f_bwd, b_bwd)}
    totals, counts = marks.totals_ms(), marks.counts()
    dom = max(totals, key=lambda x: totals[x])
    t_dom = totals[dom] / counts[dom] * 1e-3
    f_dom, b_dom = units[dom]
    roof = {"bound": "hbm", "achieved": round(b_dom / t_dom / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof.update(frac=round(roof["achieved"] / roof["peak"], 4), traffic=measured_traffic(dom, traffic_file("pma")),
                kernel=dom,
                launch_ms=round(totals[dom] / counts[dom], 4),
                algorithmic_per_launch={"flops": f_dom, "bytes": b_dom},
                other_bound_frac=round(f_dom / t_dom / 1e12 / PEAK_BF16_TFLOPS, 4))
    value = (b_fwd + b_bwd) / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": "seed pooling attention fwd+bwd, algorithmic HBM GB/s, jagged batch, 1 MI355X",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded numpy draws as in gdpa_inputs.make_pma_inputs)",
        "config": {"workload": f"seed pooling attention fwd+bwd, {m} seeds: B={B} samples, lengths "
                               f"log-normal (median {cfg.lengths[1]}, max {cfg.lengths[2]}), T={T}, H={H}, d={d}",
                   "seeds": m, "tokens": T, "heads": H, "head_dim": d, "seed": args.seed},
        "tflops": round((f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12, 2),
        "breakdown_ms_per_step": {x: round(totals[x] / args.steps, 4) for x in totals},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from oracle import pma_oracle as pmo
        chosen, toks = [], 0
        for b in range(B):
            if inp.lengths[b] == 0:
                continue
            chosen.append(b)
            toks += int(inp.lengths[b])
            if toks >= 900000:
                break
        clk = CpuClock().__enter__()
        pmo.pma_forward(inp.seeds, inp.offsets, inp.k, inp.v, samples=chosen)
        pmo.pma_backward(inp.seeds, inp.offsets, inp.k, inp.v, inp.do, samples=chosen)
        clk.__exit__(None, None, None)
        dt = clk.wall
        (_, bf), (_, bb) = pma_units(toks, len(chosen), H, d, m)
        out["cpu_baseline"] = {"value": round((bf + bb) / dt / 1e9, 3), "unit": "GB/s", **clk.fields(),
                               "kind": "oracle",
                               "sample": f"fwd+bwd on samples {chosen[0]}..{chosen[-1]} ({len(chosen)} of {B}, "
                                         f"{toks} tokens); {(bf + bb) / 1e9:.2f} GB algorithmic in {dt:.1f} s "
                                         f"(numpy float64)", "seconds": round(dt, 2)}
    print(json.dumps(out))


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        msg = ("bench.py runs on one GPU only: GDPA shards by sample with no exchange in the "
               "op itself; the benchmark measures one GPU's share. Use --gpus 1.")
        print(msg, file=sys.stderr)
        print(json.dumps({"error": msg, "n_gpus": args.gpus}))
        sys.exit(2)

    if args.record_traffic:
        record_traffic(args)
        return
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.op == "swa":
        run_swa(args)
        return
    if args.op == "pma":
        run_pma(args)
        return
    if args.op == "jagged_kv":
        run_jagged_kv(args)
        return
    if args.op == "layers":
        run_layers(args)
        return
    if args.op == "biased":
        run_biased(args)
        return
    if args.op == "grouped":
        run_grouped(args)
        return

    import numpy as np
    import torch

    import context_cross_attention_amd as cca
    import gdpa_inputs as gi
    from context_cross_attention_amd.stacked import StackedGdpa

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cca.load()
    dev = torch.device("cuda:0")
    cfg = gi.CONFIGS[args.config]
    phi = args.phi or cfg.phis[0]
    marks = Marks(torch)

    t_gen = time.perf_counter()
    rotate = 1
    if cfg.layers:
        inp = gi.make_stacked_inputs(cfg, seed=args.seed)
        T = int(inp.offsets[-1])
        x0 = inp.x0.to(dev)
        g = inp.do.to(dev)
        off = inp.offsets.to(dev)
        ctx = inp.ctx.to(dev)
        wk = [w.to(dev) for w in inp.w_k]
        wv = [w.to(dev) for w in inp.w_v]
        model = StackedGdpa(off, ctx, wk, wv, cfg.heads, cfg.n_kv, T, phi=phi)

        def step(i, mk):
            model.forward(x0, mk)
            model.backward(g, mk)
    else:
        inp = gi.make_gdpa_inputs(cfg, seed=args.seed)
        T = inp.total_tokens
        q, off, k, v = (t.to(dev) for t in (inp.q, inp.offsets, inp.k, inp.v))
        do = inp.do.to(dev) if inp.do is not None else None
        # Working sets that the 256 MB last-level cache could hold between steps are
        # rotated over enough copies (>= 1 GB in all) that every step reads from HBM.
        per_step = sum(t.numel() * t.element_size() for t in (q, k, v, q) + ((do, q, q) if do is not None else ()))
        rotate = 1 if per_step >= (512 << 20) else int(math.ceil((1 << 30) / per_step))
        sets = []
        for r in range(rotate):
            qq, kk_, vv = (t.clone() for t in (q, k, v)) if r else (q, k, v)
            sets.append(dict(q=qq, k=kk_, v=vv, do=None if do is None else (do.clone() if r else do),
                             o=torch.empty_like(q), lse=torch.empty((T, cfg.heads), dtype=torch.float32, device=dev),
                             dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v)))
        ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)

        def step(i, mk):
            z = sets[i % rotate]
            mk("gdpa_fwd", True)
            cca.fwd(z["q"], off, z["k"], z["v"], phi=phi, out=z["o"], lse=z["lse"], workspace=ws)
            mk("gdpa_fwd", False)
            if cfg.backward:
                mk("gdpa_bwd", True)
                cca.bwd(z["q"], off, z["k"], z["v"], z["o"], z["lse"], z["do"], phi=phi, dq=z["dq"], dk=z["dk"],
                        dv=z["dv"])
                mk("gdpa_bwd", False)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    print(f"# inputs ready in {t_gen:.1f} s: T={T}", file=sys.stderr, flush=True)

    def no_marks(name, start):
        return None

    # Headline: exactly `steps` steps between synchronisations, nothing else inside.
    for i in range(args.warmup):
        step(i, no_marks)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, no_marks)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    print(f"# timed {args.steps} steps: {ms_per_step:.3f} ms per step", file=sys.stderr, flush=True)

    # Statistics pass (separate from the headline): per-step HIP events and per-stage
    # events on the library's stream over >= 50 steps and >= 1 s.
    n_stats = max(50, int(math.ceil(1000.0 / max(ms_per_step, 1e-3))))
    n_stats = min(n_stats, 20000) if args.stats_steps <= 0 else args.stats_steps
    step_ev = []
    marks.enabled = True
    for i in range(n_stats):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        step(i, marks)
        e1.record()
        step_ev.append((e0, e1))
    torch.cuda.synchronize()
    marks.enabled = False
    step_ms = np.array([a.elapsed_time(b) for a, b in step_ev])

    B, H, d, n = cfg.batch, cfg.heads, cfg.head_dim, cfg.n_kv
    layers = max(cfg.layers, 1)
    fwd_f, fwd_b = gdpa_units("gdpa_fwd", T, B, H, d, n, phi, residual=bool(cfg.layers))
    bwd_f, bwd_b = gdpa_units("gdpa_bwd", T, B, H, d, n, phi)
    gdpa_flops = layers * (fwd_f + (bwd_f if cfg.backward else 0.0))
    wg_flops = 0.0
    units = {"gdpa_fwd": (fwd_f, fwd_b), "gdpa_bwd": (bwd_f, bwd_b)}
    if cfg.layers:
        cols = n * H * d
        f1, b1 = gemm_units(B, cols, cfg.ctx_dim)
        f2, b2 = gemm_units(cols, cfg.ctx_dim, B)
        units["weightgen_fwd"] = (2 * f1, 2 * b1)   # K and V per marked region
        units["weightgen_bwd"] = (2 * f2, 2 * b2)
        wg_flops = layers * 2 * (f1 + f2)
    value = gdpa_flops / (ms_per_step * 1e-3) / 1e12

    # Per-stage times: medians over the statistics steps of each stage's time per step.
    per_step_stage = {k: np.array([a.elapsed_time(b) for a, b in v]).reshape(n_stats, -1).sum(axis=1)
                      for k, v in marks.pairs.items()}
    counts = {k: len(v) // n_stats for k, v in marks.pairs.items()}
    stage_ms = {k: float(np.median(v)) for k, v in per_step_stage.items()}
    per_launch = {k: stage_ms[k] / counts[k] for k in stage_ms}
    breakdown = {k: round(v, 4) for k, v in stage_ms.items()}
    fwd_ms = stage_ms.get("gdpa_fwd", 0.0)
    bwd_ms = stage_ms.get("gdpa_bwd", 0.0)
    fwd_tflops = layers * fwd_f / (fwd_ms * 1e-3) / 1e12 if fwd_ms > 0 else None
    fwd_bwd_tflops = (layers * (fwd_f + bwd_f) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12
                      if cfg.backward and bwd_ms > 0 else None)

    dom = max(stage_ms, key=lambda k: stage_ms[k])
    f_dom, b_dom = units[dom]
    t_dom = per_launch[dom] * 1e-3
    t_mfma, t_hbm = f_dom / (PEAK_BF16_TFLOPS * 1e12), b_dom / (PEAK_HBM_GBS * 1e9)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(b_dom / t_dom / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(f_dom / t_dom / 1e12, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(dom, traffic_file((args.config, phi)))
    roof["kernel"] = dom
    roof["launch_ms"] = round(per_launch[dom], 4)
    roof["algorithmic_per_launch"] = {"flops": f_dom, "bytes": b_dom}
    roof["other_bound_frac"] = round((f_dom / t_dom / 1e12) / PEAK_BF16_TFLOPS, 4) if roof["bound"] == "hbm" \
        else round((b_dom / t_dom / 1e9) / PEAK_HBM_GBS, 4)

    if cfg.layers:
        workload = (f"stacked GDPA {cfg.layers} layers fwd+bwd incl. weight generation: B={B} samples, "
                    f"lengths log-normal (median {cfg.lengths[1]}, max {cfg.lengths[2]}), T={T}, H={H}, "
                    f"d={d}, n_kv={n}, ctx_dim={cfg.ctx_dim}, phi={phi}, residual between layers")
    else:
        workload = f"GDPA {'fwd+bwd' if cfg.backward else 'fwd'}: {cfg.name}, phi={phi}, T={T}"

    def frac(x):
        return None if x is None else round(x / PEAK_BF16_TFLOPS, 4)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy draws; lengths, values and weights as in gdpa_inputs.py)",
        "config": {"workload": workload, "global_batch": B, "tokens": T, "heads": H, "head_dim": d,
                   "n_kv": n, "layers": cfg.layers or 1, "phi": phi, "seed": args.seed},
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_tflops": None if fwd_tflops is None else round(fwd_tflops, 2),
        "fwd_frac_of_bf16_peak": frac(fwd_tflops),
        "fwd_bwd_tflops": None if fwd_bwd_tflops is None else round(fwd_bwd_tflops, 2),
        "fwd_bwd_frac_of_bf16_peak": frac(fwd_bwd_tflops),
        "gdpa_only_tflops": round(gdpa_flops / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 2),
        "gdpa_tflop_per_step": round(gdpa_flops / 1e12, 3),
        "e2e_tflops_incl_weightgen": round((gdpa_flops + wg_flops) / (ms_per_step * 1e-3) / 1e12, 2),
        "step_ms_stats": {"steps": n_stats, "median": round(float(np.median(step_ms)), 4),
                          "p10": round(float(np.percentile(step_ms, 10)), 4),
                          "p90": round(float(np.percentile(step_ms, 90)), 4),
                          "input_copies_rotated": rotate},
        "breakdown_ms_per_step": breakdown,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline_stacked(inp, cfg, phi) if cfg.layers else cpu_baseline_single(inp, cfg, phi)
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
