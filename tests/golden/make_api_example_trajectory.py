"""Writes api_example_b2_trajectory.json: the oracle's own Lloyd trajectory on
the headline recipe reduced to its first two problems (B = 2, N = 75600,
d = 128, K = 1000, fp16, tol = 1e-4, up to 100 iterations), as per-iteration
digests of the ids and counts plus the centre shift and objective.

Calls only the oracle and the seeded input generator; the GPU tests compare
the library's free-running trajectory with these digests (the oracle run
takes minutes, too long to repeat inside the GPU suite).

    python tests/golden/make_api_example_trajectory.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synthdata  # noqa: E402

OUT = os.path.join(HERE, "api_example_b2_trajectory.json")


def digest(a) -> str:
    return hashlib.sha256(np.ascontiguousarray(a, dtype="<i4").tobytes()).hexdigest()[:16]


def main():
    w = synthdata.make_workload("api_example", B=2)
    res = oracle.lloyd(w.x64(), w.init64(), 100, w.tol, w.dtype, record=True, want_near=False)
    its = []
    for t, tr in enumerate(res.trace):
        its.append({"t": t + 1, "ids": digest(tr["assign"].ids), "counts": digest(tr["counts"]),
                    "shift_max": float(tr["shift"].max()), "objective": tr["J"].tolist()})
    out = {"recipe": "api_example, B=2 (synthdata.make_workload('api_example', B=2)), "
                     "N=75600 d=128 K=1000 fp16, tol=1e-4, max_iter=100",
           "n_iter": res.n_iter, "ids_digest": "sha256 of the ids as little-endian int32, 16 hex",
           "iterations": its}
    with open(OUT, "w") as f:
        json.dump(out, f, indent=1)
    print(f"n_iter {res.n_iter}; wrote {OUT}")


if __name__ == "__main__":
    main()
