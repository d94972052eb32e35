"""Exact fp64 Gumbel-max sampling from an LM head (the plain definition).

FlashSampling (arXiv 2603.15854), Section 3:
* logits l = H W^T with H [B, D] and W [V, D] (the multi-GPU paragraph that
  opens the method introduces W in R^{V x D});
* deterministic transforms of the logits before noise (Stage 1 description);
  the only transform here is the temperature, l~ = l / T;
* Gumbel-max: s_v = l~_v + g_v with i.i.d. Gumbels g, sample = argmax_v s_v
  (the Gumbel-max paragraph);
* the fused two-stage kernel returns the same maximiser because argmax
  decomposes over vocab tiles (exactness paragraph).

Readings where the pages are silent (each listed in the design notes):
* temperature divides the logits, noise is added after (s = l/T + g); T == 0
  is greedy argmax of l;
* ties go to the lowest vocab index; NaN scores never win; a row whose
  scores are all NaN returns -1;
* accumulation is fp64 here. Products of bf16 or fp32 inputs are exact in
  fp64, so l is exact up to the fp64 summation error (about 1e-13 here).

Everything is computed from the definition, vocab chunk by vocab chunk (the
chunking only bounds memory; the maximum is taken over the whole row).
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .gumbel import gumbel_from_words
from .philox import philox_words


def _to_f64(a: np.ndarray) -> np.ndarray:
    """Widen an input array to fp64: uint16 arrays are bf16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported input dtype {a.dtype}")


def exact_logits(H: np.ndarray, W: np.ndarray, rows=None, v0: int = 0, v1=None) -> np.ndarray:
    """l[b, v] = sum_d H[b, d] W[v, d] in fp64 for the selected rows and v0 <= v < v1."""
    H = np.asarray(H)
    if H.ndim == 1:
        H = H[None, :]
    v1 = W.shape[0] if v1 is None else v1
    Hs = _to_f64(H if rows is None else H[np.asarray(rows)])
    Wc = _to_f64(W[v0:v1])
    return Hs @ Wc.T


def gumbel_noise(seed: int, step: int, rows, v0: int, v1: int) -> np.ndarray:
    """g[b, v] for the given batch rows and v0 <= v < v1 (fp64)."""
    return gumbel_from_words(philox_words(seed, step, np.asarray(rows), v0, v1))


def perturbed_scores(H, W, T: float, seed: int, step: int, rows=None, v0: int = 0,
                     v1=None) -> np.ndarray:
    """s = l / T + g (T > 0), or s = l (T == 0), fp64, shape [rows, v1 - v0]."""
    H = np.asarray(H)
    if H.ndim == 1:
        H = H[None, :]
    rows = np.arange(H.shape[0]) if rows is None else np.asarray(rows)
    v1 = W.shape[0] if v1 is None else v1
    l = exact_logits(H, W, rows, v0, v1)
    if T == 0:
        return l
    return l / np.float64(T) + gumbel_noise(seed, step, rows, v0, v1)


def argmax_lowest(s: np.ndarray, offset: int = 0) -> np.ndarray:
    """Per row of s: index of the maximum, lowest index on ties, NaN never wins.

    Returns int64 indices (plus ``offset``); -1 for a row whose entries are all NaN.
    """
    s = np.atleast_2d(np.asarray(s, dtype=np.float64))
    valid = ~np.isnan(s)
    s2 = np.where(valid, s, -np.inf)
    m = s2.max(axis=1)
    hit = valid & (s2 == m[:, None])
    idx = np.argmax(hit, axis=1).astype(np.int64) + offset
    idx[~valid.any(axis=1)] = -1
    return idx


@dataclasses.dataclass
class SampleResult:
    idx: np.ndarray      # [B] int64 sampled token (-1: all scores NaN)
    best: np.ndarray     # [B] fp64 winning perturbed score s_(1)
    second: np.ndarray   # [B] fp64 runner-up score s_(2) (-inf if V == 1)
    second_idx: np.ndarray  # [B] int64 runner-up index (-1 if none)

    @property
    def margin(self) -> np.ndarray:
        """Top-2 margin s_(1) - s_(2) per row."""
        return self.best - self.second


def _merge_top2(state, s: np.ndarray, v0: int):
    """Fold a chunk of scores (global columns v0, v0+1, ...) into the running
    per-row top-2 state (best, best_idx, second, second_idx).

    Order: higher score first, then lower vocab index; NaN never enters.
    """
    best, bidx, second, sidx = state
    n = s.shape[0]
    r = np.arange(n)
    c1 = argmax_lowest(s)
    has1 = c1 >= 0
    c1v = np.where(has1, s[r, np.maximum(c1, 0)], -np.inf)
    rest = s.copy()
    rest[r[has1], c1[has1]] = np.nan  # remove the chunk winner, then take the next
    c2 = argmax_lowest(rest)
    has2 = c2 >= 0
    c2v = np.where(has2, s[r, np.maximum(c2, 0)], -np.inf)
    vals = np.stack([best, second, c1v, c2v], axis=1)
    idxs = np.stack([bidx, sidx, np.where(has1, c1 + v0, -1), np.where(has2, c2 + v0, -1)], axis=1)
    present = idxs >= 0
    # sort each row's four candidates by (score descending, index ascending);
    # absent entries sort last
    order = np.lexsort((np.where(present, idxs, np.iinfo(np.int64).max),
                        np.where(present, -vals, np.inf)), axis=1)
    v_sorted = np.take_along_axis(np.where(present, vals, -np.inf), order, axis=1)
    i_sorted = np.take_along_axis(np.where(present, idxs, -1), order, axis=1)
    return v_sorted[:, 0], i_sorted[:, 0], v_sorted[:, 1], i_sorted[:, 1]


def sample(H, W, T: float, seed: int, step: int, rows=None, vocab_chunk: int = 8192) -> SampleResult:
    """Gumbel-max sample per batch row over the whole vocabulary, with top-2.

    ``rows`` selects batch rows of H (their row index is the Philox row); by
    default every row. The result is the plain definition: argmax of
    s = l / T + g over all V, lowest index on ties.
    """
    H = np.asarray(H)
    if H.ndim == 1:
        H = H[None, :]
    rows = np.arange(H.shape[0]) if rows is None else np.asarray(rows)
    V = W.shape[0]
    n = len(rows)
    state = (np.full(n, -np.inf), np.full(n, -1, dtype=np.int64),
             np.full(n, -np.inf), np.full(n, -1, dtype=np.int64))
    for v0 in range(0, V, vocab_chunk):
        v1 = min(V, v0 + vocab_chunk)
        s = perturbed_scores(H, W, T, seed, step, rows, v0, v1)
        state = _merge_top2(state, s, v0)
    best, bidx, second, sidx = state
    return SampleResult(bidx, best, second, sidx)


def sample_two_stage(H, W, T: float, seed: int, step: int, tile_bounds, rows=None) -> np.ndarray:
    """The pages' two-stage form: per vocab tile a tile-local maximiser (Stage 1),
    then an argmax over the tile candidates (Stage 2).

    ``tile_bounds`` is an increasing list [0 = t_0 < t_1 < ... < t_n = V] of
    tile edges (tiles may be ragged). Returns [B] int64 indices.
    """
    H = np.asarray(H)
    if H.ndim == 1:
        H = H[None, :]
    rows = np.arange(H.shape[0]) if rows is None else np.asarray(rows)
    s = perturbed_scores(H, W, T, seed, step, rows)
    cand_score = []
    cand_idx = []
    for a, b in zip(tile_bounds[:-1], tile_bounds[1:]):
        i = argmax_lowest(s[:, a:b], offset=a)
        sc = np.where(i >= 0, s[np.arange(len(rows)), np.maximum(i, 0)], np.nan)
        cand_score.append(sc)
        cand_idx.append(i)
    cs = np.stack(cand_score, axis=1)
    ci = np.stack(cand_idx, axis=1)
    out = np.empty(len(rows), dtype=np.int64)
    for r in range(len(rows)):
        best = None
        for sc, ix in zip(cs[r], ci[r]):
            if ix < 0 or np.isnan(sc):
                continue
            if best is None or sc > best[0] or (sc == best[0] and ix < best[1]):
                best = (sc, ix)
        out[r] = -1 if best is None else best[1]
    return out
