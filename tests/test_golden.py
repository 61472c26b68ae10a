"""The oracle still reproduces its frozen tiny fixtures, and the scalar brute force agrees."""
import json
import os

import numpy as np
import pytest

from oracle import gdpa_oracle as orc
from oracle.brute import brute_forward

HERE = os.path.dirname(os.path.abspath(__file__))


def load_cases():
    with open(os.path.join(HERE, "golden", "tiny_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", load_cases(), ids=lambda c: c["name"])
def test_golden_case(case):
    q, k, v, do = (np.array(case[x]) for x in ("q", "k", "v", "do"))
    off = np.array(case["offsets"])
    o, lse = orc.gdpa_forward(q, off, k, v, case["phi"], case["scale"])
    assert np.abs(o - np.array(case["o"])).max() <= 1e-14
    if lse is not None:
        assert np.abs(lse - np.array(case["lse"])).max() <= 1e-14
    dq, dk, dv = orc.gdpa_backward(q, off, k, v, do, case["phi"], case["scale"])
    for got, key in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        assert np.abs(got - np.array(case[key])).max() <= 1e-13
    scale = case["scale"] if case["scale"] is not None else orc.default_scale(case["phi"], case["d"])
    ob, _ = brute_forward(q.tolist(), off.tolist(), k.tolist(), v.tolist(), case["phi"], scale)
    assert np.abs(np.array(ob) - np.array(case["o"])).max() <= 1e-13
