"""32-bit word -> uniform on (0, 1) -> standard Gumbel, in fp64.

The pages draw i.i.d. standard Gumbel noise (FlashSampling, Section 3, the
Gumbel-max paragraph); they do not say how. The reading adopted here:

* u = (x + 1/2) * 2^-32 for a 32-bit word x. This is exact in fp64 and lies
  strictly inside (0, 1), so no epsilon is needed: u ranges over
  [2^-33, 1 - 2^-33].
* g = -ln(-ln u), the inverse of the Gumbel CDF F(g) = exp(-exp(-g)).

For u > 1/2 the inner log is evaluated as -log1p(-(1 - u)) with 1 - u
formed exactly, which keeps full relative precision where the largest
Gumbels (the ones that decide the sample) live.
"""
from __future__ import annotations

import numpy as np

TWO_M32 = 2.0 ** -32


def word_to_uniform(x) -> np.ndarray:
    """u = (x + 0.5) * 2^-32 in fp64 (exact)."""
    return (np.asarray(x, dtype=np.float64) + 0.5) * TWO_M32


def uniform_to_gumbel(u) -> np.ndarray:
    """g = -ln(-ln u) for u in (0, 1), fp64."""
    u = np.asarray(u, dtype=np.float64)
    e = np.where(u <= 0.5, -np.log(u), -np.log1p(-(1.0 - u)))
    return -np.log(e)


def gumbel_from_words(x) -> np.ndarray:
    """Gumbel noise for 32-bit words x (any integer array), fp64."""
    x = np.asarray(x, dtype=np.uint64)
    # 1 - u = (2^32 - x - 0.5) * 2^-32, formed exactly from the integer.
    u = word_to_uniform(x)
    one_minus_u = (np.float64(2.0 ** 32) - x.astype(np.float64) - 0.5) * TWO_M32
    e = np.where(u <= 0.5, -np.log(u), -np.log1p(-one_minus_u))
    return -np.log(e)
