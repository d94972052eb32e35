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


def check_grouped_parity(H, W, T, seed, step, group_size, rows, gpu_tokens, tol=TOL, ref=None):
    """Compare GPU tokens of the grouped variant with oracle.sample_grouped.

    A row must match index-exactly when both the group draw (top-2 margin of
    the group scores m_k + h_k) and the local sample inside the chosen group
    (top-2 margin of the perturbed scores) clear TOL. Otherwise the GPU token's
    group must score within TOL of the best group, and the token's perturbed
    score within TOL of its group's best. Returns (n_rows, n_near_ties).
    """
    rows = np.asarray(rows)
    gpu_tokens = np.asarray(gpu_tokens).astype(np.int64)
    if ref is None:
        ref = oracle.sample_grouped(H, W, T, seed, step, group_size, rows=rows)
    gm, lm = ref.group_margin, ref.local_margin
    near = 0
    for k, b in enumerate(rows):
        g = int(gpu_tokens[k])
        if gm[k] > tol and lm[k] > tol:
            assert g == ref.idx[k], (f"row {b}: gpu {g} != oracle {ref.idx[k]} (group margin {gm[k]:.3e}, "
                                     f"local margin {lm[k]:.3e}, G={group_size}, T={T}, seed={seed}, step={step})")
            continue
        near += 1
        assert 0 <= g < W.shape[0], f"row {b}: gpu token {g} out of range"
        kg = g // group_size
        t = np.where(np.isnan(ref.group_score[k]), -np.inf, ref.group_score[k])
        if T != 0:
            assert t[kg] >= t.max() - tol, f"row {b}: gpu group {kg} scores {t[kg]} < best {t.max()} - {tol}"
        s = oracle.perturbed_scores(H, W, T, seed, step, rows=[b], v0=g, v1=g + 1)[0, 0]
        assert s >= ref.local_best[k, kg] - tol, (f"row {b}: gpu token {g} scores {s} < its group's best "
                                                  f"{ref.local_best[k, kg]} - {tol}")
    return len(rows), near
