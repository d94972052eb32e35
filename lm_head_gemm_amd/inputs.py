"""Seeded synthetic inputs for the fused LM-head sampler (recipe "FS-DATA-1").

This module holds no arithmetic of the sampling method: it only draws the
hidden states H [B_max, D] and LM-head weights W [V, D] that both the HIP path
and the CPU oracle consume, so that the two sides provably see identical bits.

Recipe (the pages give no input values; trained LM heads are replaced by
Gaussian heads of the same shapes):

* ``ss = SeedSequence(seed)``; ``kH, kW, kS = ss.spawn(3)``.
* H = standard normal float32 [B_max, D] drawn from ``default_rng(kH)``.
* W = sigma * standard normal float32, drawn in consecutive blocks of
  ``W_BLOCK_ROWS`` vocab rows; block i uses ``default_rng(kW.spawn(n)[i])``
  so blocks can be drawn on several threads without changing the stream.
* bf16 inputs are the round-to-nearest-even bf16 of those float32 values
  (stored here as their uint16 bit patterns); fp32 inputs stay float32.
* Optionally a seeded fraction of vocab rows (``round(frac * V)`` rows chosen
  without replacement by ``default_rng(kS)``) is multiplied by ``row_scale``
  after rounding (x4 is exact in bf16), which makes some logits peaked.

H for a batch B is the first B rows of H, so a smaller batch is a prefix of a
larger one.
"""
from __future__ import annotations

import dataclasses
import hashlib
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

W_BLOCK_ROWS = 8192


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic LM-head workload."""

    name: str
    D: int
    V: int
    dtype: str  # "bf16" or "f32"
    sigma_w: float
    temperature: float
    seed: int
    batches: tuple
    scaled_frac: float = 0.0
    row_scale: float = 1.0
    steps: tuple = (0,)
    vocab_tile: int | None = None

    @property
    def b_max(self) -> int:
        return max(self.batches)


# The five workloads. Shapes follow public LM heads (Llama-3-8B, Qwen-7B,
# 70B-class, DeepSeek-V3); the values are synthetic.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", D=256, V=4096, dtype="f32", sigma_w=0.05,
                         temperature=1.0, seed=0, batches=(1,),
                         steps=tuple(range(64)), vocab_tile=256),
    "llama3_8b": Workload("llama3_8b", D=4096, V=128256, dtype="bf16", sigma_w=0.02,
                          temperature=1.0, seed=1, batches=(1, 8, 32, 64, 128, 256)),
    "qwen_7b": Workload("qwen_7b", D=3584, V=152064, dtype="bf16", sigma_w=0.02,
                        temperature=0.7, seed=2, batches=(1, 4, 16, 64, 256)),
    "llama3_70b": Workload("llama3_70b", D=8192, V=128256, dtype="bf16", sigma_w=0.015,
                           temperature=1.0, seed=3, batches=(1, 16, 64, 256, 512)),
    "deepseek_v3": Workload("deepseek_v3", D=7168, V=129280, dtype="bf16", sigma_w=0.015,
                            temperature=0.6, seed=4, batches=(1, 64, 256, 1024),
                            scaled_frac=0.01, row_scale=4.0),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_hidden(wl: Workload, b_max: int | None = None) -> np.ndarray:
    """H [b_max, D]: uint16 bf16 bits, or float32 for fp32 workloads."""
    b_max = wl.b_max if b_max is None else b_max
    kH, _, _ = np.random.SeedSequence(wl.seed).spawn(3)
    h = np.random.default_rng(kH).standard_normal((b_max, wl.D), dtype=np.float32)
    return h if wl.dtype == "f32" else f32_to_bf16_bits(h)


def make_weights(wl: Workload, v_rows: int | None = None) -> np.ndarray:
    """W [V, D] (or its first v_rows rows): uint16 bf16 bits, or float32."""
    V = wl.V
    nblk = (V + W_BLOCK_ROWS - 1) // W_BLOCK_ROWS
    _, kW, kS = np.random.SeedSequence(wl.seed).spawn(3)
    kids = kW.spawn(nblk)
    rows = V if v_rows is None else min(V, v_rows)
    out_dtype = np.float32 if wl.dtype == "f32" else np.uint16
    W = np.empty((rows, wl.D), dtype=out_dtype)
    sigma = np.float32(wl.sigma_w)

    def fill(i: int) -> None:
        r0 = i * W_BLOCK_ROWS
        if r0 >= rows:
            return
        n = min(W_BLOCK_ROWS, V - r0)
        x = np.random.default_rng(kids[i]).standard_normal((n, wl.D), dtype=np.float32)
        x *= sigma
        take = min(n, rows - r0)
        W[r0:r0 + take] = x[:take] if wl.dtype == "f32" else f32_to_bf16_bits(x[:take])

    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(fill, range(nblk)))

    if wl.scaled_frac > 0.0:
        sel = scaled_rows(wl)
        sel = sel[sel < rows]
        if wl.dtype == "f32":
            W[sel] *= np.float32(wl.row_scale)
        else:
            W[sel] = f32_to_bf16_bits(bf16_bits_to_f32(W[sel]) * np.float32(wl.row_scale))
    return W


def scaled_rows(wl: Workload) -> np.ndarray:
    """Sorted indices of the vocab rows that are scaled by ``row_scale``."""
    if wl.scaled_frac <= 0.0:
        return np.zeros(0, dtype=np.int64)
    _, _, kS = np.random.SeedSequence(wl.seed).spawn(3)
    n = int(round(wl.scaled_frac * wl.V))
    return np.sort(np.random.default_rng(kS).choice(wl.V, n, replace=False))


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()


def chi2_inputs(seed: int = 0):
    """Small fp32 head for the sampling-distribution test: h [256], W [64, 256].

    h ~ N(0, 1), W ~ N(0, 0.05^2), both float32.
    """
    kh, kw = np.random.SeedSequence(seed).spawn(2)
    h = np.random.default_rng(kh).standard_normal(256, dtype=np.float32)
    w = np.random.default_rng(kw).standard_normal((64, 256), dtype=np.float32) * np.float32(0.05)
    return h, w
