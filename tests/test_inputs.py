"""Seeded synthetic inputs: reproducible, correctly shaped, with the stated length laws."""
import numpy as np
import torch

import gdpa_inputs as gi


def test_lengths_seed0_totals():
    # Total tokens at seed 0 for the four jagged workloads.
    want = {2: 144490, 3: 383345, 4: 304653, 5: 1438675}
    for i, total in want.items():
        cfg = gi.CONFIGS[i]
        L = gi.draw_lengths(np.random.default_rng(0), cfg.lengths, cfg.batch)
        assert L.sum() == total
        spec = cfg.lengths
        if spec[0] == "uniform":
            assert L.min() >= spec[1] and L.max() <= spec[2]
        else:
            assert L.min() >= 1 and L.max() <= spec[2]


def test_inputs_deterministic_and_shaped():
    cfg = gi.small_config(gi.CONFIGS[4], batch=3, lengths=("uniform", 2, 9))
    a = gi.make_gdpa_inputs(cfg, seed=5)
    b = gi.make_gdpa_inputs(cfg, seed=5)
    assert torch.equal(a.q, b.q) and torch.equal(a.k, b.k) and torch.equal(a.do, b.do)
    T = a.total_tokens
    assert a.q.shape == (T, 4, 128) and a.k.shape == (3, 1024, 4, 128)
    assert a.q.dtype == torch.bfloat16 and a.offsets.dtype == torch.int32
    assert a.offsets[0] == 0 and int(a.offsets[-1]) == T


def test_stacked_inputs():
    cfg = gi.small_config(gi.CONFIGS[5], batch=4, lengths=("uniform", 1, 5), layers=2)
    s = gi.make_stacked_inputs(cfg, seed=0)
    assert len(s.w_k) == 2 and s.w_k[0].shape == (256 * 8 * 128, 512)
    a = gi.xavier_uniform_bound(512, 256 * 8 * 128)
    assert float(s.w_k[0].float().abs().max()) <= a * 1.01
