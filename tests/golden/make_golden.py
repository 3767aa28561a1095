"""Write tests/golden/oracle_small.json: a small fixed case and the oracle's answer.

Calls only oracle/ (and numpy).  The pages print no worked example of
attention outputs, so this fixture is a regression anchor for the oracle
itself; the oracle is pinned independently by tests/test_oracle.py.
Run:  python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle  # noqa: E402


def main():
    rng = np.random.default_rng(20261203)
    q = rng.standard_normal((1, 4, 5, 4)).round(3)
    k = rng.standard_normal((1, 2, 7, 4)).round(3)
    v = rng.standard_normal((1, 2, 7, 4)).round(3)
    sinks = np.array([0.5, -1.25, 20.0, 3.0])
    window, scale = 4, 0.5
    o, l = oracle.attention_fwd(q, k, v, sinks, window, scale)
    out = dict(q=q.tolist(), k=k.tolist(), v=v.tolist(), sinks=sinks.tolist(), window=window,
               scale=scale, out=o.tolist(), lse=l.tolist())
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
