"""The oracle reproduces its frozen result on the seeded tiny decode workload
(tests/golden/make_golden.py wrote the fixture from the oracle alone)."""
import json
import os

import numpy as np

from tests.golden.make_golden import compute

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_frozen_tiny_decode():
    with open(os.path.join(HERE, "golden", "tiny_decode_oracle.json")) as f:
        ref = json.load(f)
    w, o, lse = compute()
    assert [int(x) for x in w.kv_len] == ref["kv_len"], "input generator changed"
    assert abs(float(w.q.double().sum()) - ref["q_sum"]) < 1e-9, "input generator changed"
    np.testing.assert_allclose(lse, np.array(ref["lse"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[:, :, :8], np.array(ref["o_first8"]), rtol=0, atol=1e-12)
