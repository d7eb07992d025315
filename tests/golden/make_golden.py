"""Writes tests/golden/tiny_oracle.json from the fp64 oracle alone.

The documentation pages print no worked example with values, so the only
stored expectations are the oracle's own results on the seeded tiny
workload (2 rows, H=16, page_size 16, kv lens 37 and 100, query lens 1
and 5, causal).  They anchor later runs against accidental changes to the
oracle and give the GPU smoke check a fixed target.

Run from the repository root:  python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

COLS = list(range(0, 512, 37))


def main():
    w = workloads.tiny()
    o, lse = oracle.attention(w.q_nope, w.q_pe, w.kv_cache, w.qo_indptr, w.kv_indptr,
                              w.kv_indices, w.kv_last_page_len, w.page_size, w.causal,
                              w.sm_scale)
    doc = {
        "workload": "tiny (seed 1001): B=2, H=16, page_size=16, kv lens 37/100, "
                    "qo lens 1/5, causal, sm_scale=fp32(192**-0.5)",
        "source": "fp64 oracle (oracle/mla_oracle.py), written by tests/golden/make_golden.py",
        "cols": COLS,
        "lse": lse.tolist(),
        "o_cols": o[:, :, COLS].tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=0)
        f.write("\n")


if __name__ == "__main__":
    main()
