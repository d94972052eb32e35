"""Every row of every batch size of the four LM-head workloads at their full
sizes, against the CPU oracle (FlashSampling, arXiv 2603.15854, Section 3,
exactness paragraph: the fused kernel returns the maximiser a full Gumbel-max
pass computes).

H for a batch B is the first B rows of the workload's H and a row's noise is
keyed by its row index, so one oracle pass over the largest batch of a
workload gives the expected token, best score and top-2 margin of every row of
every smaller batch. Each batch is then run in every launch configuration the
benchmark times (row-major W and the tiled layout, two-stage and single-pass,
the unfused baseline with fp32 logits, a ragged vocab tile at small B) and
every row of every one is held to the parity rule of tests/_util.py.

With FS_PARITY_RECORD set to a file path, the row counts and the near-tie
fraction of each workload are merged into that JSON file.
"""
import json
import os
import time

import numpy as np
import pytest

import oracle
from lm_head_gemm_amd import inputs
from tests._util import TOL, check_grouped_parity, check_parity, to_device

pytestmark = pytest.mark.gpu

FULL = ["llama3_8b", "qwen_7b", "llama3_70b", "deepseek_v3"]


@pytest.fixture(scope="module")
def fs():
    import torch
    assert torch.cuda.is_available()
    from lm_head_gemm_amd import flashsample
    return flashsample


def _record(name, entry):
    path = os.environ.get("FS_PARITY_RECORD")
    if not path:
        return
    rec = {}
    if os.path.exists(path):
        with open(path) as f:
            rec = json.load(f)
    rec[name] = entry
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)


def _prefix(ref, B):
    return oracle.SampleResult(ref.idx[:B], ref.best[:B], ref.second[:B], ref.second_idx[:B])


@pytest.fixture(scope="module", params=FULL)
def full(request, fs):
    import torch
    wl = inputs.WORKLOADS[request.param]
    t0 = time.perf_counter()
    H = inputs.make_hidden(wl)
    W = inputs.make_weights(wl)
    t1 = time.perf_counter()
    ref = oracle.sample(H, W, wl.temperature, wl.seed, 0)
    t2 = time.perf_counter()
    print(f"\n[{wl.name}] inputs {t1 - t0:.1f} s, oracle over {H.shape[0]} rows {t2 - t1:.1f} s", flush=True)
    Hd, Wd = to_device(H), to_device(W)
    tw = fs.TiledWeights(Wd)
    yield wl, H, W, ref, Hd, Wd, tw, t2 - t1
    del Hd, Wd, tw
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_full_size_every_row(fs, full):
    """All rows of every B of the workload's sweep plus B = 4 (the four-row
    GEMV plan on row-major heads 4096 to 8192 wide), in each launch
    configuration; launch configurations agree with one another on every row
    where the oracle's margin decides the token."""
    import torch
    wl, H, W, ref, Hd, Wd, tw, oracle_s = full
    T, seed = wl.temperature, wl.seed
    batches = sorted(set(wl.batches) | {4})
    checks = {}
    near_checks = 0
    for B in batches:
        sub = _prefix(ref, B)
        Hb = Hd[:B]
        toks = {
            "rows": fs.sample_fused(Hb, Wd, T, seed, 0),
            "rows-single": fs.sample_fused(Hb, Wd, T, seed, 0, single_pass=True),
            "tiled": fs.sample_fused(Hb, tw, T, seed, 0),
            "tiled-single": fs.sample_fused(Hb, tw, T, seed, 0, single_pass=True),
            "unfused-f32-tiled": fs.sample_unfused(Hb, tw, T, seed, 0, logits_dtype=torch.float32),
        }
        if B <= 16:
            # a vocab tile that does not divide V: the last tile is ragged
            assert wl.V % 1008 != 0
            toks["rows-gemv-1008"] = fs.sample_fused(Hb, Wd, T, seed, 0, variant="gemv", vocab_tile=1008)
        for name, tok in toks.items():
            tok = tok.cpu().numpy()
            assert tok.min() >= 0 and tok.max() < wl.V, (B, name)
            n, k = check_parity(H, W, T, seed, 0, np.arange(B), tok, ref=sub)
            checks[f"B{B}/{name}"] = n
            near_checks += k
    n_checks = sum(checks.values())
    assert n_checks == sum(B * (5 + (B <= 16)) for B in batches)
    near_rows = int(np.sum(ref.margin <= TOL))
    frac = near_rows / len(ref.idx)
    print(f"[{wl.name}] {n_checks} row checks over B={batches}; near-tie rows {near_rows}/{len(ref.idx)} "
          f"({frac:.4f}); min margin {float(np.min(ref.margin)):.3e}", flush=True)
    _record(wl.name, {"D": wl.D, "V": wl.V, "T": T, "seed": seed, "step": 0, "batches": batches,
                      "oracle_rows": int(len(ref.idx)), "near_tie_rows": near_rows, "near_tie_fraction": frac,
                      "tolerance": TOL, "row_checks": n_checks, "near_tie_row_checks": near_checks,
                      "checks": checks, "oracle_seconds": round(oracle_s, 1),
                      "min_margin": float(np.min(ref.margin))})


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,batches,G", [("llama3_8b", (64, 256), 16384), ("deepseek_v3", (16, 64), 1024)])
def test_grouped_full_size_every_row(fs, name, batches, G):
    """The grouped variant at full size: every row of each batch (smaller
    batches are prefixes, so one oracle pass serves all), on the tiled layout
    the benchmark times and on row-major W."""
    wl = inputs.WORKLOADS[name]
    B_max = max(batches)
    H = inputs.make_hidden(wl)[:B_max]
    W = inputs.make_weights(wl)
    t = time.perf_counter()
    ref = oracle.sample_grouped(H, W, wl.temperature, wl.seed, 3, G)
    print(f"\n[{name} grouped G={G}] oracle over {B_max} rows {time.perf_counter() - t:.1f} s", flush=True)
    Hd, Wd = to_device(H), to_device(W)
    tw = fs.TiledWeights(Wd)
    total = near = 0
    for B in batches:
        sub = oracle.GroupedResult(ref.idx[:B], ref.group[:B], ref.group_score[:B], ref.mass[:B],
                                   ref.local_idx[:B], ref.local_best[:B], ref.local_second[:B])
        for Wx in (tw, Wd):
            tok = fs.sample_fused(Hd[:B], Wx, wl.temperature, wl.seed, 3, group_size=G).cpu().numpy()
            assert tok.min() >= 0 and tok.max() < wl.V
            n, k = check_grouped_parity(H, W, wl.temperature, wl.seed, 3, G, np.arange(B), tok, ref=sub)
            total += n
            near += k
    assert total == 2 * sum(batches)
    print(f"[{name} grouped G={G}] {total} row checks, {near} near ties", flush=True)
    _record(f"{name}/grouped_G{G}", {"batches": list(batches), "group_size": G, "step": 3, "row_checks": total,
                                     "near_tie_row_checks": near})
