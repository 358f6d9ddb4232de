"""Writes tests/golden/tiny_f32_rows.json from the CPU oracle alone.

Fixture: the tiny fp32 workload (1 sequence, L=256, 4 index heads x 32,
top-64, 4-head MLA 80/64, seed 0) through the oracle's whole path on a few
query rows, rows 0..63 being the dense-vs-sparse crossover (fewer than 64
previous tokens).  Stored per row: the selected index set (sorted), the lse of
each head, and the sum over value columns of each head's output.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import get, make_inputs  # noqa: E402

ROWS = [0, 1, 31, 62, 63, 64, 65, 127, 200, 255]


def main():
    wl = get("tiny_f32")
    inp = make_inputs(wl)
    res = oracle.forward(inp, wl, rows=ROWS)
    g = {
        "workload": wl.name,
        "source": "oracle.forward on workloads.make_inputs(tiny_f32, cpu, seed 0)",
        "rows": ROWS,
        "idx_sorted": {str(r): sorted(int(x) for x in res["idx"][i] if x >= 0) for i, r in enumerate(ROWS)},
        "lse": {str(r): [float(v) for v in res["lse"][i]] for i, r in enumerate(ROWS)},
        "out_rowsum": {str(r): [float(v) for v in res["out"][i].sum(axis=-1)] for i, r in enumerate(ROWS)},
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_f32_rows.json")
    with open(path, "w") as f:
        json.dump(g, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
