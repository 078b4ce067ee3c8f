"""Writes tests/golden/oracle_small.json: regression outputs of the CPU oracle on tiny
seeded inputs.  Calls only oracle/ (and numpy for the inputs)."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import oracle  # noqa: E402


def main():
    cases = []
    for n, (shape, causal, scale) in enumerate([((1, 2, 5, 3), 1, 0.5), ((2, 1, 4, 2), 0, 1.25)]):
        rng = np.random.default_rng(500 + n)
        q, k, v = (np.round(rng.standard_normal(shape), 3) for _ in range(3))
        O, L = oracle.attention(q, k, v, causal, scale)
        cases.append(dict(shape=shape, causal=causal, scale=scale, q=q.tolist(), k=k.tolist(),
                          v=v.tolist(), O=O.tolist(), lse=L.tolist()))
    with open(os.path.join(HERE, "oracle_small.json"), "w") as f:
        json.dump({"written_by": "tests/golden/make_oracle_fixtures.py", "cases": cases}, f, indent=1)


if __name__ == "__main__":
    main()
