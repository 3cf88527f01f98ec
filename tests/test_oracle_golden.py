"""The oracle reproduces its stored regression fixture bit for bit."""
import json
import os

import numpy as np

from tests.golden import make_golden


def test_oracle_matches_stored_fixture():
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_e4m3_oracle.json")
    with open(path) as f:
        doc = json.load(f)
    w, c, out, lse = make_golden.compute()
    assert doc["spec"] == make_golden.SPEC
    assert out.view(np.uint32).reshape(-1).tolist() == doc["out_bits"]
    assert lse.view(np.uint32).reshape(-1).tolist() == doc["lse_bits"]
    assert int(np.uint32(np.frombuffer(c.k.tobytes(), np.uint8).astype(np.uint64).sum())) == doc["k_codes_crc"]
