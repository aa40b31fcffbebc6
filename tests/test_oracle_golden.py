"""Regression lock on the oracle (tests/golden/oracle_tiny.json, written by make_golden.py)."""
import json
import os

import numpy as np

from recsys_jagged_attention_gdpa_amd import synth
from tests.helpers import oracle_bwd, oracle_fwd

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_stored_tiny_output():
    with open(os.path.join(HERE, "golden", "oracle_tiny.json")) as f:
        g = json.load(f)
    w = synth.make(g["workload"])
    assert w.q_off.tolist() == g["q_offsets"]
    got = oracle_fwd(w)
    got.update(oracle_bwd(w))
    for name in ("o", "dq", "dk", "dv"):
        for r, row in g[name].items():
            assert np.allclose(got[name][int(r)], np.asarray(row), rtol=1e-13, atol=1e-13), name
        assert abs(got[name].sum() - g[name + "_sum"]) <= 1e-10 * max(1.0, abs(g[name + "_sum"]))
