"""Host-side logic of the benchmark, no GPU: the FLOP accounting of the layer
stack agrees with the oracle's own count, the window pair count is the brute-force
count, a committed counter record is used only while its kernel sources are
unchanged, and a multi-GPU request exits with a message before touching a GPU."""
import json
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
    rec = {"kernels": {"gdpa_bwd": {"bytes_per_launch": 123, "source_sha256": bench.kernel_source_hash("gdpa_bwd")},
                       "gdpa_fwd": {"bytes_per_launch": 456, "source_sha256": "0" * 64}}}
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(rec))
    assert bench.measured_traffic("gdpa_bwd", str(p)) == 123
    assert bench.measured_traffic("gdpa_fwd", str(p)) is None      # sources changed since
    assert bench.measured_traffic("weightgen_fwd", str(p)) is None  # no reading
    assert bench.measured_traffic("gdpa_bwd", str(tmp_path / "missing.json")) is None
    # Each call hashes only its own kernels' sources (and the shared headers).
    assert bench.kernel_source_hash("gdpa_bwd") != bench.kernel_source_hash("pma_bwd")


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["n_gpus"] == 2 and "one GPU" in out["error"]
