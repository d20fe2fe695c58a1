"""Writes tests/golden/oracle_small_f32.json: a small f32 workload run through
the CPU oracle only (routing, alignment at block_m=4, FFN output). It guards
the oracle against accidental change; it is not a pin by itself (the pins are
the brute-force, closed-form, invariant and library tests).

Run from the repository root: python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from synth import make_inputs, fingerprint  # noqa: E402

CASE = dict(T=5, E=8, H=64, I=32, k=2, dtype="f32", routing="router", seed=0, wstd=0.05)


def compute():
    inp = make_inputs(CASE["T"], CASE["E"], CASE["H"], CASE["I"], CASE["k"], dtype="f32",
                      routing="router", seed=0, device="cpu", wstd=0.05)
    ids, w = oracle.route(inp.host_logits(), CASE["k"])
    s, b, n = oracle.align(ids, CASE["E"], 4)
    out = oracle.ffn(inp.host_x().astype(np.float64),
                     lambda e: inp.host_w1(e).astype(np.float64),
                     lambda e: inp.host_w2(e).astype(np.float64), ids, w)
    return dict(case=CASE, inputs_sha256=fingerprint(inp), topk_ids=ids.tolist(),
                topk_weights=w.tolist(), sorted_ids=s.tolist(), block_expert=b.tolist(),
                num_padded=int(n), out=out.tolist())


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small_f32.json")
    with open(path, "w") as f:
        json.dump(compute(), f)
    print("wrote", path)
