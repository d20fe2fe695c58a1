"""The oracle still reproduces the fixture its own committed script wrote."""
import json
import os

import numpy as np

from tests.golden.make_golden import compute

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_reproduces_golden_fixture():
    with open(os.path.join(HERE, "golden", "oracle_small_f32.json")) as f:
        ref = json.load(f)
    got = compute()
    assert got["inputs_sha256"] == ref["inputs_sha256"]
    for key in ("topk_ids", "sorted_ids", "block_expert", "num_padded"):
        assert got[key] == ref[key], key
    assert np.allclose(got["topk_weights"], ref["topk_weights"], rtol=1e-15, atol=0)
    assert np.allclose(got["out"], ref["out"], rtol=1e-13, atol=1e-15)
