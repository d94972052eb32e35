"""The stored oracle outputs under tests/golden/ still follow from the oracle
and the seeded inputs (the file is written by tests/golden/make_golden.py)."""
import os

import numpy as np

import oracle
from lm_head_gemm_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_tiny_tokens():
    rows = []
    shas = {}
    with open(os.path.join(GOLDEN, "tiny_f32_tokens.txt")) as f:
        for line in f:
            if line.startswith("# H sha256") or line.startswith("# W sha256"):
                shas[line.split()[1]] = line.split()[3]
            elif not line.startswith("#"):
                p = line.split()
                rows.append((int(p[0]), int(p[1]), float(p[2]), float(p[3]), int(p[4])))
    return rows, shas


def test_tiny_inputs_checksums():
    wl = inputs.WORKLOADS["tiny_f32"]
    _, shas = load_tiny_tokens()
    assert inputs.sha256(inputs.make_hidden(wl)) == shas["H"]
    assert inputs.sha256(inputs.make_weights(wl)) == shas["W"]


def test_tiny_tokens_reproduce():
    wl = inputs.WORKLOADS["tiny_f32"]
    H, W = inputs.make_hidden(wl), inputs.make_weights(wl)
    rows, _ = load_tiny_tokens()
    assert len(rows) == 64
    for step, tok, best, margin, second in rows:
        r = oracle.sample(H, W, wl.temperature, wl.seed, step)
        assert int(r.idx[0]) == tok and int(r.second_idx[0]) == second
        assert np.isclose(r.best[0], best, rtol=0, atol=1e-12)
        assert np.isclose(r.margin[0], margin, rtol=0, atol=1e-12)
