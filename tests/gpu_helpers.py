"""Shared helpers for the GPU parity tests: run the HIP path and the fp64 oracle
on the same seeded inputs and compare with the max-abs-relative metric."""
from __future__ import annotations

import sys

import numpy as np
import torch

import gdpa_inputs as gi
from oracle import gdpa_oracle as orc

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def max_abs_rel(gpu, ref) -> float:
    """max |gpu - ref| / max |ref| over one output tensor (NaN entries of ref skipped)."""
    g = gpu.detach().float().cpu().double().numpy() if hasattr(gpu, "detach") else np.asarray(gpu)
    r = np.asarray(ref, dtype=np.float64)
    mask = ~np.isnan(r)
    if not mask.any():
        return 0.0
    den = np.abs(r[mask]).max()
    if den == 0:
        return float(np.abs(g[mask]).max())
    return float(np.abs(g[mask] - r[mask]).max() / den)


def custom_config(lengths, H, d, n, dtype="bf16", phi="softmax", backward=True):
    return gi.GdpaConfig(f"custom L={list(lengths)[:6]} H={H} d={d} n={n}", len(lengths), H, d, n,
                         ("explicit", list(lengths)), dtype, (phi,), backward=backward)


def device_inputs(inp: gi.GdpaInputs, dev="cuda"):
    return (inp.q.to(dev), inp.offsets.to(dev), inp.k.to(dev), inp.v.to(dev),
            None if inp.do is None else inp.do.to(dev))
