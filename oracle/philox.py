"""Philox4x32-10 counter-based generator, written from its published definition.

Source: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3", SC'11, Section 4 (the Philox S-box / bijection
and its key schedule). One call maps a 128-bit counter (four 32-bit words)
and a 64-bit key (two words) to four 32-bit output words through 10 rounds.

Round (counter c0..c3, key k0, k1):
    (hi0, lo0) = M0 * c0      (full 64-bit product of two 32-bit words)
    (hi1, lo1) = M1 * c2
    c' = (hi1 ^ c1 ^ k0,  lo1,  hi0 ^ c3 ^ k1,  lo0)
and between rounds the key is bumped by the Weyl constants (k0 += W0,
k1 += W1, mod 2^32). The multipliers and Weyl constants are the ones the
paper gives for Philox4x32.

Sampler keying (the pages name no generator; noise only has to be i.i.d. and
a function of position): key = (seed mod 2^32, seed >> 32); counter =
(v >> 2, row, step mod 2^32, step >> 32); the Gumbel for vocab index v uses
output word v & 3.

Two implementations live here: a vectorised numpy one (uint64 lanes holding
32-bit words) and a scalar Python-int one used only to cross-check the
vectorised code on small inputs.
"""
from __future__ import annotations

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF
ROUNDS = 10


def philox4x32_10_scalar(ctr, key):
    """One Philox4x32-10 call on Python ints. ctr: 4 words, key: 2 words."""
    c0, c1, c2, c3 = (int(x) & MASK32 for x in ctr)
    k0, k1 = (int(x) & MASK32 for x in key)
    for r in range(ROUNDS):
        if r:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0, p1 & MASK32,
                          (p0 >> 32) ^ c3 ^ k1, p0 & MASK32)
    return (c0, c1, c2, c3)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10. Arguments broadcast; returns four uint64 arrays
    holding the 32-bit output words."""
    m32 = np.uint64(MASK32)
    sh = np.uint64(32)
    c0, c1, c2, c3, k0, k1 = np.broadcast_arrays(
        *(np.asarray(x, dtype=np.uint64) & m32 for x in (c0, c1, c2, c3, k0, k1)))
    c0, c1, c2, c3 = (x.copy() for x in (c0, c1, c2, c3))
    k0 = k0.copy()
    k1 = k1.copy()
    M0 = np.uint64(PHILOX_M0)
    M1 = np.uint64(PHILOX_M1)
    W0 = np.uint64(PHILOX_W0)
    W1 = np.uint64(PHILOX_W1)
    for r in range(ROUNDS):
        if r:
            k0 = (k0 + W0) & m32
            k1 = (k1 + W1) & m32
        p0 = M0 * c0  # < 2^64: exact in uint64
        p1 = M1 * c2
        c0, c1, c2, c3 = ((p1 >> sh) ^ c1 ^ k0, p1 & m32,
                          (p0 >> sh) ^ c3 ^ k1, p0 & m32)
    return c0, c1, c2, c3


def philox_words(seed: int, step: int, row, v0: int, v1: int) -> np.ndarray:
    """The 32-bit words for vocab indices v0 <= v < v1 of the given row(s).

    ``row`` may be an int or a 1-D array of rows; the result has shape
    [len(rows), v1 - v0] (or [v1 - v0] for an int row), dtype uint64.
    """
    scalar_row = np.ndim(row) == 0
    rows = np.atleast_1d(np.asarray(row, dtype=np.uint64))
    q0, q1 = v0 >> 2, (v1 + 3) >> 2
    quads = np.arange(q0, q1, dtype=np.uint64)
    seed = int(seed)
    step = int(step)
    out = philox4x32_10(quads[None, :], rows[:, None],
                        step & MASK32, (step >> 32) & MASK32,
                        seed & MASK32, (seed >> 32) & MASK32)
    words = np.stack(out, axis=-1).reshape(len(rows), -1)  # word j of quad q -> 4q + j
    words = words[:, v0 - 4 * q0: v1 - 4 * q0]
    return words[0] if scalar_row else words
