"""Grouped (hierarchical) exact sampling, fp64: per vocabulary group a local
sample and a local log-mass, then a categorical choice of the group.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FlashSampling (arXiv 2603.15854): in the tensor-parallel paragraphs of
Section 3 each vocabulary shard returns a local sample and a local log-mass
instead of its logits; the abstract states that such grouped variants are
exact by hierarchical factorisation of the categorical distribution.

Readings adopted where the pages are silent:
* groups are contiguous vocabulary ranges of ``group_size`` entries: group k
  covers [k G, min((k + 1) G, V)); the last one may be shorter;
* local sample x_k: the Gumbel-max over the group with the token noise g of
  the plain sampler, argmax_{v in group k} (l_v / T + g_v), lowest index on
  ties, NaN never wins;
* local log-mass m_k = log sum_{v in group k} exp(l_v / T) over the group's
  non-NaN entries (-inf for a group with none);
* group choice: Gumbel-max over the log-masses with its own noise stream,
  t_k = m_k + h_k, k* = argmax_k t_k (lowest k on ties). h_k comes from the
  same Philox4x32-10 key with counter (0xC0000000 | k >> 2, row, step mod
  2^32, step >> 32), word k & 3, and the same word -> uniform -> Gumbel map.
  Token noise uses counter word 0 = v >> 2 < 2^29, so the two streams never
  share a counter;
* the sample is x_{k*}; T == 0 is the greedy argmax of l (the limit).

Why it is exact: for token v in group k,
  P(sample = v) = P(k* = k) P(x_k = v)
               = (e^{m_k} / sum_j e^{m_j}) (e^{l_v / T} / e^{m_k}),
which is softmax(l / T)_v. The chosen token generally differs from the plain
sampler's for the same seed (the group draw uses other noise); agreement is in
distribution, and index-exact only in the two reductions tested: one group
(the plain sample) and groups of one token (a plain sample with the group
noise).
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .gumbel import gumbel_from_words
from .philox import philox4x32_10
from .sampler import argmax_lowest, exact_logits, gumbel_noise

GROUP_COUNTER_TAG = 0xC0000000
_MASK32 = 0xFFFFFFFF


def group_philox_words(seed: int, step: int, rows, k0: int, k1: int) -> np.ndarray:
    """Group-stream words for groups k0 <= k < k1 of each row: uint64 [len(rows), k1 - k0]."""
    rows = np.atleast_1d(np.asarray(rows, dtype=np.uint64))
    q0, q1 = k0 >> 2, (k1 + 3) >> 2
    quads = np.arange(q0, q1, dtype=np.uint64) | np.uint64(GROUP_COUNTER_TAG)
    seed, step = int(seed), int(step)
    out = philox4x32_10(quads[None, :], rows[:, None], step & _MASK32, (step >> 32) & _MASK32,
                        seed & _MASK32, (seed >> 32) & _MASK32)
    words = np.stack(out, axis=-1).reshape(len(rows), -1)
    return words[:, k0 - 4 * q0: k1 - 4 * q0]


def group_noise(seed: int, step: int, rows, n_groups: int) -> np.ndarray:
    """h[b, k] for the given rows and groups 0 <= k < n_groups (fp64)."""
    return gumbel_from_words(group_philox_words(seed, step, rows, 0, n_groups))


def log_mass(x: np.ndarray) -> np.ndarray:
    """log sum exp over the last axis, skipping NaN; -inf when nothing is left."""
    x = np.asarray(x, dtype=np.float64)
    ok = ~np.isnan(x)
    xm = np.where(ok, x, -np.inf)
    m = xm.max(axis=-1)
    finite = np.isfinite(m)
    shift = np.where(finite, m, 0.0)
    e = np.where(ok, np.exp(xm - shift[..., None]), 0.0)
    with np.errstate(divide="ignore"):   # an empty sum is replaced below
        out = shift + np.log(e.sum(axis=-1))
    out = np.where(finite, out, m)   # all -inf (or none left): -inf; a +inf entry: +inf
    return out


@dataclasses.dataclass
class GroupedResult:
    idx: np.ndarray           # [n] sampled token (-1: no non-NaN candidate)
    group: np.ndarray         # [n] chosen group k*
    group_score: np.ndarray   # [n, K] t_k = m_k + h_k (NaN for T == 0)
    mass: np.ndarray          # [n, K] local log-mass m_k
    local_idx: np.ndarray     # [n, K] local sample x_k
    local_best: np.ndarray    # [n, K] s at x_k
    local_second: np.ndarray  # [n, K] runner-up s inside the group (-inf if none)

    @property
    def group_margin(self) -> np.ndarray:
        """Top-2 margin of the group scores per row (inf with one group)."""
        t = np.where(np.isnan(self.group_score), -np.inf, self.group_score)
        if t.shape[1] < 2:
            return np.full(t.shape[0], np.inf)
        top = -np.sort(-t, axis=1)
        return top[:, 0] - top[:, 1]

    @property
    def local_margin(self) -> np.ndarray:
        """Top-2 margin of the perturbed scores inside the chosen group."""
        r = np.arange(len(self.idx))
        return self.local_best[r, self.group] - self.local_second[r, self.group]


def _top2_in(s: np.ndarray, offset: int):
    """Per row: (index of the max, its score, the second score) with the plain
    sampler's order (higher score, then lower index; NaN never enters)."""
    i1 = argmax_lowest(s, offset=offset)
    r = np.arange(s.shape[0])
    has = i1 >= 0
    best = np.where(has, s[r, np.maximum(i1 - offset, 0)], -np.inf)
    rest = s.copy()
    rest[r[has], (i1 - offset)[has]] = np.nan
    i2 = argmax_lowest(rest)
    second = np.where(i2 >= 0, s[r, np.maximum(i2, 0)], -np.inf)
    return i1, best, second


def sample_grouped(H, W, T: float, seed: int, step: int, group_size: int, rows=None) -> GroupedResult:
    """The grouped sample of each selected batch row of H (row index = Philox row)."""
    if group_size <= 0:
        raise ValueError("group_size must be positive")
    H = np.asarray(H)
    if H.ndim == 1:
        H = H[None, :]
    rows = np.arange(H.shape[0]) if rows is None else np.asarray(rows)
    V = W.shape[0]
    n = len(rows)
    K = (V + group_size - 1) // group_size
    l = exact_logits(H, W, rows)
    if T == 0:
        s = l
        lt = None
    else:
        lt = l / np.float64(T)
        s = lt + gumbel_noise(seed, step, rows, 0, V)
    local_idx = np.empty((n, K), dtype=np.int64)
    local_best = np.empty((n, K))
    local_second = np.empty((n, K))
    mass = np.full((n, K), np.nan)
    for k in range(K):
        a, b = k * group_size, min(V, (k + 1) * group_size)
        local_idx[:, k], local_best[:, k], local_second[:, k] = _top2_in(s[:, a:b], a)
        if lt is not None:
            mass[:, k] = log_mass(lt[:, a:b])
    r = np.arange(n)
    if T == 0:
        # the T -> 0 limit: the group holding the global maximiser
        g_idx = argmax_lowest(l)
        group = np.where(g_idx >= 0, g_idx // group_size, 0)
        return GroupedResult(g_idx, group, np.full((n, K), np.nan), mass, local_idx, local_best, local_second)
    t = mass + group_noise(seed, step, rows, K)
    group = argmax_lowest(t)
    group = np.where(group >= 0, group, 0)
    return GroupedResult(local_idx[r, group], group, t, mass, local_idx, local_best, local_second)
