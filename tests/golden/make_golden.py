"""Write tests/golden/tiny_cases.json from the fp64 oracle (calls only oracle/).

The pages print no worked numerical example for GDPA, so these fixtures freeze
the oracle's own outputs on tiny jagged batches (including an empty sample and
n not a power of two).  A later change to the oracle's arithmetic shows up as a
mismatch here and has to be justified by a passage of the pages.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle import gdpa_oracle as orc  # noqa: E402

CASES = [
    # name, lengths, H, d, n, phi, scale (None = default), seed
    ("softmax_ragged", [3, 0, 5], 2, 4, 3, "softmax", None, 101),
    ("silu_ragged", [1, 4, 0, 2], 1, 4, 5, "silu", None, 102),
    ("softmax_scaled", [6], 2, 2, 7, "softmax", 0.75, 103),
]


def main():
    out = []
    for name, lengths, H, d, n, phi, scale, seed in CASES:
        rng = np.random.default_rng(seed)
        T, B = sum(lengths), len(lengths)
        off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
        q = np.round(rng.standard_normal((T, H, d)), 3)
        k = np.round(rng.standard_normal((B, n, H, d)), 3)
        v = np.round(rng.standard_normal((B, n, H, d)), 3)
        do = np.round(rng.standard_normal((T, H, d)), 3)
        o, lse = orc.gdpa_forward(q, off, k, v, phi, scale)
        dq, dk, dv = orc.gdpa_backward(q, off, k, v, do, phi, scale)
        out.append(dict(name=name, phi=phi, scale=scale, offsets=off.tolist(), H=H, d=d, n=n,
                        q=q.tolist(), k=k.tolist(), v=v.tolist(), do=do.tolist(),
                        o=o.tolist(), lse=None if lse is None else lse.tolist(),
                        dq=dq.tolist(), dk=dk.tolist(), dv=dv.tolist()))
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_cases.json")
    with open(path, "w") as f:
        json.dump({"generator": "tests/golden/make_golden.py (fp64 oracle)", "cases": out}, f)
    print("wrote", path)


if __name__ == "__main__":
    main()
