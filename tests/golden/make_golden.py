"""Writes the stored expected values under tests/golden/ from the CPU oracle.

Only the seeded input generator and the oracle are called. Run from the
repository root:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from lm_head_gemm_amd import inputs  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def tiny_f32_tokens():
    wl = inputs.WORKLOADS["tiny_f32"]
    H = inputs.make_hidden(wl)
    W = inputs.make_weights(wl)
    lines = ["# tiny fp32 head: B=1, D=256, V=4096, T=1.0, seed=0, steps 0..63",
             "# H sha256 " + inputs.sha256(H), "# W sha256 " + inputs.sha256(W),
             "# step token best_score margin runner_up"]
    for step in wl.steps:
        r = oracle.sample(H, W, wl.temperature, wl.seed, step)
        lines.append(f"{step} {int(r.idx[0])} {float(r.best[0])!r} {float(r.margin[0])!r} {int(r.second_idx[0])}")
    with open(os.path.join(HERE, "tiny_f32_tokens.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    tiny_f32_tokens()
