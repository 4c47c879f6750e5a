"""Writes dropout_gap.json: for each rate p (the pages' 0.05 and 0.1, and
0.3), a seed and a flat element index of X whose Philox4x32-10 word lies
between the float64 and the float32 readings of the drop threshold, i.e. in
[floor(p * 2^32), floor(fl32(p) * 2^32)). The library takes the rate as a
float, so that element is dropped; a float64 rate would keep it. The search
calls only the oracle's generator.

    python tests/golden/dropout_gap.py
"""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from oracle import dropout as od  # noqa: E402

RATES = (0.05, 0.1, 0.3)
M, K = 300, 512          # the search stays inside an M x K activation


def search(p):
    lo = int(np.floor(p * 4294967296.0))       # float64 reading
    hi = od.drop_threshold(p)                  # float32 reading (the library's)
    assert hi > lo
    for seed in range(1, 1 << 20):
        w = od.philox_words(seed, 0, M * K).astype(np.int64)
        hit = np.flatnonzero((w >= lo) & (w < hi))
        if hit.size:
            e = int(hit[0])
            return {"p": p, "seed": seed, "index": e, "word": int(w[e]), "thr_f64": lo,
                    "thr_f32": hi, "M": M, "k": K}
    raise SystemExit(f"no seed found for p = {p}")


def main():
    cases = [search(p) for p in RATES]
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "dropout_gap.json")
    with open(path, "w") as f:
        json.dump(cases, f, indent=1)
    for c in cases:
        print(c)


if __name__ == "__main__":
    main()
