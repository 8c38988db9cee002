"""Write the stored expected values under tests/golden/ — calls only the oracle.

The pages print no worked numeric example of attention, so no fixture here is
a value from the pages; each file is the oracle's output on a seeded workload,
kept so that a silent change of the generator or the oracle shows up as a
diff.  Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import oracle as OR  # noqa: E402
from paged_kv_attention_prefill_amd import workloads as W  # noqa: E402


def summary(w):
    o, lse, mx = OR.attention(w)
    return {
        "workload": w.manifest(),
        "lse": lse.round(15).tolist(),
        "max": mx.round(15).tolist(),
        "o_first2": o[..., :2].round(15).tolist(),
        "o_rowsum": o.sum(-1).round(15).tolist(),
        "o_rownorm": np.sqrt((o * o).sum(-1)).round(15).tolist(),
    }


def main():
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c1_tiny_decode_oracle.json")
    with open(out, "w") as f:
        json.dump(summary(W.config1()), f, indent=1)
    print("wrote", out)


if __name__ == "__main__":
    main()
