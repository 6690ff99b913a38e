"""Writes oracle_tiny.json: the float64 oracle's output on the tiny workload
(B1 T64 H4 W16, fp32 N(0,1), seed 1), as a regression record.

Calls only the oracle and the seeded input generator.  Re-run it only when a
change to the oracle's arithmetic is justified by a reading of the pages, and
say which in the commit message.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from sliding_window_attention_vx_amd import synth  # noqa: E402


def main():
    c = synth.CONFIGS["tiny"]
    x = synth.make_config("tiny")
    o = oracle.prefill(x["q"], x["k"], x["v"], c.W, theta=c.theta)
    rec = {
        "workload": "tiny: B1 T64 H4 D64 W16 theta 1e6, fp32 N(0,1), seed 1, positions 0..63",
        "input_sha256": {k: synth.sha256(x[k]) for k in ("q", "k", "v")},
        "sum": float(o.sum()),
        "sum_sq": float((o * o).sum()),
        "samples": {f"{t},{h},{d}": float(o[0, t, h, d])
                    for (t, h, d) in [(0, 0, 0), (15, 1, 31), (16, 2, 32), (63, 3, 63), (40, 0, 7)]},
    }
    with open(os.path.join(os.path.dirname(__file__), "oracle_tiny.json"), "w") as f:
        json.dump(rec, f, indent=1)


if __name__ == "__main__":
    main()
