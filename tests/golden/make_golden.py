"""Write tests/golden/tiny_case.json: a tiny EFLA case computed by the fp64 oracle only.

It is a regression fixture (it catches accidental changes to the oracle); the
oracle's correctness is pinned by tests/test_oracle_pins.py against independent
references. Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle import efla_oracle as O  # noqa: E402


def main():
    r = np.random.default_rng(42)
    B, H, T, dk, dv = 1, 2, 7, 3, 2
    inp = dict(q=r.standard_normal((B, H, T, dk)), k=r.standard_normal((B, H, T, dk)) * 1.7,
               v=r.standard_normal((B, H, T, dv)), beta=r.uniform(0.0, 1.0, (B, H, T)),
               do=r.standard_normal((B, H, T, dv)))
    scale = 0.75
    o, _ = O.forward(inp["q"], inp["k"], inp["v"], inp["beta"], scale=scale)
    g = O.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["do"], scale=scale)
    out = dict(note="EFLA oracle output for a tiny seeded case (seed 42); written by make_golden.py",
               scale=scale, inputs={n: x.tolist() for n, x in inp.items()}, o=o.tolist(),
               **{n: g[n].tolist() for n in ("dq", "dk", "dv", "dbeta")})
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_case.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
