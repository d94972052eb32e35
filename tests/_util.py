"""Shared helpers for the GPU tests: device upload of the seeded inputs and the
parity rule between the HIP path and the oracle.

Parity rule (floating point decides the sampled index): on every row whose
oracle top-2 margin s_(1) - s_(2) exceeds TOL, the GPU token equals the oracle
token; on rows at or below TOL, the oracle's own score of the GPU token lies
within TOL of the oracle's best score. TOL = 1e-3 is far above the GPU's
rounding error (fp32 accumulation of bf16 products plus fp32 noise, about
1e-5 at the largest configurations).
"""
from __future__ import annotations

import numpy as np

import oracle

TOL = 1e-3


def to_device(a: np.ndarray, device="cuda"):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def check_parity(H, W, T, seed, step, rows, gpu_tokens, tol=TOL, ref=None):
    """Compare GPU tokens for the given batch rows with the oracle.

    ``ref`` may hold a precomputed oracle.sample result for exactly ``rows``.
    Returns (n_rows, n_near_ties). Raises AssertionError with details on a
    violation.
    """
    rows = np.asarray(rows)
    gpu_tokens = np.asarray(gpu_tokens).astype(np.int64)
    if ref is None:
        ref = oracle.sample(H, W, T, seed, step, rows=rows)
    near = 0
    for k, b in enumerate(rows):
        g = int(gpu_tokens[k])
        if ref.margin[k] > tol:
            assert g == ref.idx[k], (f"row {b}: gpu {g} != oracle {ref.idx[k]} "
                                     f"(margin {ref.margin[k]:.3e}, T={T}, seed={seed}, step={step})")
        else:
            near += 1
            assert 0 <= g < W.shape[0], f"row {b}: gpu token {g} out of range"
            s = oracle.perturbed_scores(H, W, T, seed, step, rows=[b], v0=g, v1=g + 1)[0, 0]
            assert s >= ref.best[k] - tol, (f"row {b}: near-tie but gpu token {g} scores {s} "
                                            f"< best {ref.best[k]} - {tol}")
    return len(rows), near
