"""Write oracle regression values for a few rows of the tiny fp32 workload.

Calls only oracle/ (and the seeded inputs of workloads/).  Run from the repo
root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import attention_jvp_head  # noqa: E402
from workloads import WORKLOADS, head_array  # noqa: E402

ROWS = [0, 1, 63, 64, 127]


def main():
    w = WORKLOADS["tiny_self_fp32"]
    out = {"workload": w.name, "rows": ROWS, "heads": []}
    for h in range(w.H):
        a = {t: head_array(w, t, 0, h) for t in ("q", "k", "v", "tq", "tk", "tv")}
        O, tO, lse = attention_jvp_head(a["q"], a["k"], a["v"], a["tq"], a["tk"], a["tv"], w.scale, rows=ROWS)
        out["heads"].append({"b": 0, "h": h, "O": O.tolist(), "tO": tO.tolist(), "lse": lse.tolist()})
    with open(os.path.join(HERE, "oracle_tiny_self_fp32_rows.json"), "w") as f:
        json.dump(out, f)


if __name__ == "__main__":
    main()
