"""Host-side logic of the benchmark, no GPU: the FLOP accounting of the layer
stack agrees with the oracle's own count, the window pair count is the brute-force
count, a committed counter record is used only while its kernel sources are
unchanged, and a multi-GPU request exits with a message before touching a GPU."""
import json
import time
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from oracle import compskip_oracle as cso

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("schedule", ["full", "compskip"])
def test_layer_stack_flops_match_oracle_count(schedule):
    lengths = [130, 0, 257, 33, 600, 1]
    a = bench.layer_stack_flops(lengths, 2, 64, 64, 64, 8, 40, 4, schedule)
    b = cso.flops(lengths, 2, 64, 64, 64, 8, 40, 4, schedule)
    for k in ("gdpa", "weightgen", "hsp", "sa", "total"):
        assert a[k] == pytest.approx(b[k], rel=1e-12), k


@pytest.mark.parametrize("w", [1, 3, 7, 50])
def test_window_pairs_brute_force(w):
    lengths = [0, 1, 5, 12, 40]
    brute = sum(1 for L in lengths for i in range(L) for j in range(L) if i - w < j <= i)
    assert bench.swa_pairs(lengths, w) == brute


def test_pooling_units_count_every_tensor_once():
    T, B, H, d, m = 1000, 3, 2, 64, 32
    (ff, fb), (bf, bb) = bench.pma_units(T, B, H, d, m)
    assert ff == 4 * m * d * H * T and bf == 10 * m * d * H * T
    tok, pooled = T * H * d * 2, B * m * H * d * 2
    assert fb == 2 * tok + pooled + m * H * d * 2 + B * m * H * 4          # K, V, O, seeds, LSE
    assert bb == 4 * tok + 2 * pooled + 2 * m * H * d * 2 + B * m * H * 4  # + dK, dV, dO, dSeeds


def test_counter_record_tied_to_sources(tmp_path):
    srcs = ["gdpa_bwd_res.hip", "gdpa_sched.hip"]
    rec = {"kernels": {"gdpa_bwd": {"bytes_per_launch": 123, "sources": srcs, "source_sha256": bench.source_hash(srcs)},
                       "gdpa_fwd": {"bytes_per_launch": 456, "sources": ["gdpa_fwd_res.hip"], "source_sha256": "0" * 64},
                       "pma_fwd": {"bytes_per_launch": 789, "source_sha256": bench.source_hash([])}}}
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(rec))
    assert bench.measured_traffic("gdpa_bwd", str(p)) == 123
    assert bench.measured_traffic("gdpa_fwd", str(p)) is None      # sources changed since
    assert bench.measured_traffic("pma_fwd", str(p)) is None       # record names no sources
    assert bench.measured_traffic("weightgen_fwd", str(p)) is None  # no reading
    assert bench.measured_traffic("gdpa_bwd", str(tmp_path / "missing.json")) is None
    assert bench.measured_traffic("gdpa_bwd", None) is None
    # Each call hashes only its own kernels' sources (and the shared headers).
    assert bench.source_hash(srcs) != bench.source_hash(["gdpa_pma.hip", "gdpa_sched.hip"])


def test_traffic_records_are_per_workload():
    # A workload without a record of its own never borrows another's reading.
    assert bench.traffic_file((5, "softmax")) is None
    assert bench.traffic_file((4, "silu")) is None
    for key in bench.TRAFFIC_FILES:
        path = bench.traffic_file(key)
        assert os.path.exists(path), path
        with open(path) as f:
            rec = json.load(f)
        for stage, k in rec["kernels"].items():
            assert k["sources"] and k["bytes_per_launch"] > 0, (key, stage)


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["n_gpus"] == 2 and "one GPU" in out["error"]


def test_cpu_clock_counts_the_cores_a_region_keeps_busy():
    # One busy thread for ~0.3 s: about one core; the CPU model is read from the host.
    with bench.CpuClock() as clk:
        t0 = time.perf_counter()
        x = 0
        while time.perf_counter() - t0 < 0.3:
            x += 1
    f = clk.fields()
    assert 0.5 <= f["cores_effective"] <= 1.5 and f["cores"] == 1
    assert f["processes"] == 1 and f["threads_available"] >= 1 and isinstance(f["cpu_model"], str)


def test_traffic_record_rewrite(tmp_path):
    # Two synthetic rocprofv3 counter CSVs (two dispatches per kernel, the second
    # reading twice the first) rewrite a copy of the committed stacked-workload record:
    # every stage's bytes are its kernels' mean readings scaled by the record's copy
    # calibration, and the record ties itself to the current sources.
    import csv
    import shutil
    src = os.path.join(ROOT, "profiles", "traffic_stacked_b1024_h8_d128_n256_silu.json")
    path = tmp_path / "rec.json"
    shutil.copy(src, path)
    rec = json.load(open(src))
    names = {"bwd_res_kernel<1, 1>": "void gdpa::bwd_res_kernel<1, 1>(gdpa::BwdArgs)",
             "fwd_res_kernel<128, 256, 1, 1>": "void gdpa::fwd_res_kernel<128, 256, 1, 1>(gdpa::FwdArgs, int const*)",
             "gemm_nt_kernel": "gdpa::gemm_nt_kernel(int, long, int, unsigned short const*)",
             "gemm_tn_kernel": "gdpa::gemm_tn_kernel(int, long, int, unsigned short const*)"}
    base = {n: 1000.0 * (i + 1) for i, n in enumerate(names)}
    for counter, sub, mult in (("FETCH_SIZE", "f", 1.0), ("WRITE_SIZE", "w", 3.0)):
        d = tmp_path / sub / "host" / "123"
        d.mkdir(parents=True)
        with open(d / "run_counter_collection.csv", "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            did = 0
            for rep in (1, 2):
                for n, full in names.items():
                    did += 1
                    w.writerow([did, full, counter, base[n] * mult * rep])
                    w.writerow([did, full, "OTHER", 7.0])
    bench.rewrite_traffic_record(str(path), str(tmp_path / "f"), str(tmp_path / "w"), "--record-traffic f w")
    out = json.load(open(path))
    cal = rec["calibration"]
    for stage, k in out["kernels"].items():
        fetch = sum(1.5 * base[n] for n in k["kernels"])
        write = sum(4.5 * base[n] for n in k["kernels"])
        assert k["fetch_kib"] == pytest.approx(fetch)
        assert k["write_kib"] == pytest.approx(write)
        assert k["bytes_per_launch"] == round((fetch * cal["fetch_scale"] + write * cal["write_scale"]) * 1024)
        assert k["source_sha256"] == bench.source_hash(k["sources"])
    md = open(tmp_path / "rec.md").read()
    assert "--record-traffic f w" in md and "| gdpa_bwd |" in md
