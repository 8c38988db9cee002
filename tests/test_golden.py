"""Regression check: the seeded config-1 workload and the oracle still give the
stored values (tests/golden/c1_tiny_decode_oracle.json, written by
tests/golden/make_golden.py, which calls only the oracle)."""
import json
import os

import numpy as np

from oracle import oracle as OR
from paged_kv_attention_prefill_amd import workloads as W

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                    "c1_tiny_decode_oracle.json")


def test_config1_matches_stored_oracle_values():
    g = json.load(open(GOLD))
    w = W.config1()
    assert w.manifest() == g["workload"]
    o, lse, mx = OR.attention(w)
    np.testing.assert_allclose(lse, g["lse"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(mx, g["max"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(o[..., :2], g["o_first2"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(o.sum(-1), g["o_rowsum"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(np.sqrt((o * o).sum(-1)), g["o_rownorm"], rtol=1e-13, atol=1e-14)
