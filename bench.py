"""Benchmark of the fused LM-head sampler on one MI355X.

A step is one fused sampling call (Stage 1 + Stage 2) over one batch of
synthetic hidden states against a resident LM head. Default workload: the
Llama-3-8B-shaped head (D=4096, V=128256, bf16) at B=64, with W held in the
tiled matrix-core layout (repacked once, before timing; --layout rows times
the row-major path). Prints ONE JSON line with samples/s, the Stage-1
kernel's achieved HBM bandwidth against MI355X's 8 TB/s (and its counter-
measured traffic when profiles/ holds a record for these sources), and
beside them: single-pass, the grouped variant, the unfused baseline (bf16 and
fp32 logits) with the IO model's prediction, the row-major layout, and the
CPU oracle's rate. After the headline, a compact sweep (`sweep`) times every
workload at every B of its sweep (fewer calls per point): the fused call,
its Stage-1 HBM and matrix-core fractions, the row-major call, single-pass
at B <= 8, the unfused baseline, the store-logits overhead against the IO
model and the library GEMM alone. --sweep adds every B of the headline
workload with the headline's full detail.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--batch B] [--sweep]
                  [--layout auto|tiled|rows] [--group-size G] [--probe] [--graph]
                  [--no-all-sweep] [--sweep-steps K] [--sweep-repeats R]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_F32_PEAK_TFLOPS = 157.3   # dense fp32 matrix peak (fp32 heads run v_mfma_f32_16x16x4_f32)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The sources the timed Stage-1 kernel (tiled layout) and its launch are built
# from: a traffic record is valid only while they are unchanged.
STAGE1_SOURCES = ("include/flashsample.h", "lm_head_gemm_amd/csrc/fs_common.h",
                  "lm_head_gemm_amd/csrc/stage1_tiled.hip", "lm_head_gemm_amd/csrc/api.hip")


def code_of(text: str) -> str:
    """C/C++ source without comments and blank space: what the compiler sees."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(read=None) -> str:
    """Hash of the code (comments and layout ignored) of STAGE1_SOURCES:
    identifies the kernel a traffic record belongs to."""
    h = hashlib.sha256()
    for f in STAGE1_SOURCES:
        if read is None:
            with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
                text = fh.read()
        else:
            text = read(f)
        h.update(f.encode() + code_of(text).encode())
    return h.hexdigest()[:16]


def upload(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def stage1_bytes(B, D, V, esz, n_tiles) -> int:
    """Algorithmic bytes of one Stage-1 launch: W read once, H read once, one
    8-byte candidate written per (row, vocab tile)."""
    return V * D * esz + B * D * esz + 8 * B * n_tiles


def warm(fn, warmup, min_ms):
    """Runs fn(i) for `warmup` untimed steps and, further, until at least
    min_ms of wall time has passed (clocks settle after tens of ms of load)."""
    import torch
    i = 0
    t0 = time.perf_counter()
    while i < warmup or (time.perf_counter() - t0) * 1e3 < min_ms:
        fn(i)
        i += 1
        if i % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


def roofline(rec, mfma_peak, traffic):
    """Roofline block for the Stage-1 kernel: HBM-bound while its arithmetic
    intensity (2BVD flops over its algorithmic bytes) is below the ridge
    peak flops / 8 TB/s, matrix-core bound above it."""
    ai = rec["flops"] / rec["stage1_bytes"]
    ridge = mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    common = {"traffic": traffic, "kernel": "stage1 (fused GEMM + Gumbel-max epilogue)",
              "stage1_us": rec["stage1_ms"] * 1e3, "flop_per_byte": ai, "ridge_flop_per_byte": ridge}
    if ai <= ridge:
        return {"bound": "hbm", "achieved": rec["stage1_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": rec["stage1_GBps"] / HBM_PEAK_GBS, **common}
    return {"bound": "mfma", "achieved": rec["stage1_TFLOPs"], "peak": mfma_peak, "unit": "TFLOP/s",
            "frac": rec["stage1_TFLOPs"] / mfma_peak, **common}


def time_fused(fs, Hb, Ws, wl, steps, warmup, B, variant="auto", vocab_tile=0, batch_tile=0,
               single_pass=False, min_warm_ms=0.0, group_size=0, repeats=1, runs_out=None):
    """Returns (ms per step, median Stage-1 ms, warm-up steps run).

    The step time comes from `steps` back-to-back calls bracketed by two
    events (with repeats > 1: the median of that many such runs, whose
    per-step times are appended to runs_out); the Stage-1 time from passes
    of `steps` calls in which the library records an event pair around each
    Stage-1 launch on the same stream (those extra records are kept out of
    the step time). Timed runs and Stage-1 passes alternate, so both see the
    same clocks while the part heats up under a long matrix-core load."""
    import torch
    T, seed = wl.temperature, wl.seed
    tiled = isinstance(Ws[0], fs.TiledWeights)
    ws = torch.empty(fs.workspace_bytes(B, wl.D, wl.V, Hb.dtype, variant=variant, vocab_tile=vocab_tile,
                                        tiled=tiled, single_pass=single_pass, group_size=group_size,
                                        batch_tile=batch_tile),
                     dtype=torch.uint8, device="cuda")
    if single_pass:
        fs.workspace_reset(ws)
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    kw = dict(out=out, workspace=ws, variant=variant, vocab_tile=vocab_tile, batch_tile=batch_tile,
              single_pass=single_pass, group_size=group_size)
    n_warm = warm(lambda i: fs.sample_fused(Hb, Ws[i % len(Ws)], T, seed, i, **kw), warmup, min_warm_ms)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:  # create the HIP events; the library re-records them around Stage 1
        a.record()
        b.record()
    runs, s1s = [], []
    for _ in range(max(1, repeats)):
        torch.cuda.synchronize()
        t0.record()
        for i in range(steps):
            fs.sample_fused(Hb, Ws[i % len(Ws)], T, seed, i, **kw)
        t1.record()
        torch.cuda.synchronize()
        runs.append(t0.elapsed_time(t1) / steps)
        for i in range(steps):
            fs.sample_fused(Hb, Ws[i % len(Ws)], T, seed, i, events=ev[i], **kw)
        torch.cuda.synchronize()
        s1s.extend(a.elapsed_time(b) for a, b in ev)
    if runs_out is not None:
        runs_out.extend(runs)
    s1 = float(np.median(s1s))   # robust to a stray slow record
    return float(np.median(runs)), s1, n_warm


def time_unfused(fs, Hb, Ws, wl, steps, warmup, B, logits_dtype, min_warm_ms=0.0):
    import torch
    ws = torch.empty(fs.unfused_workspace_bytes(B, wl.D, wl.V, Hb.dtype, logits_dtype), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    warm(lambda i: fs.sample_unfused(Hb, Ws[i % len(Ws)], wl.temperature, wl.seed, i, logits_dtype, out=out,
                                     workspace=ws), warmup, min_warm_ms)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        fs.sample_unfused(Hb, Ws[i % len(Ws)], wl.temperature, wl.seed, i, logits_dtype, out=out, workspace=ws)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def time_interleaved(calls, steps, repeats, warm_ms):
    """Median ms per call of each callable in `calls` (each takes the step
    index), measured in alternating runs of `steps` calls so that every
    variant sees the same clocks and temperature; returns a list."""
    import torch
    for fn in calls:
        warm(fn, 3, warm_ms / max(1, len(calls)))
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    runs = [[] for _ in calls]
    for _ in range(max(1, repeats)):
        for k, fn in enumerate(calls):
            torch.cuda.synchronize()
            t0.record()
            for i in range(steps):
                fn(i)
            t1.record()
            torch.cuda.synchronize()
            runs[k].append(t0.elapsed_time(t1) / steps)
    return [float(np.median(r)) for r in runs]


def io_model_calls(fs, Hb, Ws, wl, B):
    """The three calls of the IO-model check on one batch: the fused call,
    the fused call that also stores bf16 logits, and the unfused baseline
    (bf16 logits written, then read back by the sampler)."""
    import torch
    T, seed = wl.temperature, wl.seed
    tiled = isinstance(Ws[0], fs.TiledWeights)
    ws = torch.empty(fs.workspace_bytes(B, wl.D, wl.V, Hb.dtype, tiled=tiled), dtype=torch.uint8, device="cuda")
    uws = torch.empty(fs.unfused_workspace_bytes(B, wl.D, wl.V, Hb.dtype, torch.bfloat16), dtype=torch.uint8,
                      device="cuda")
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    logits = torch.empty((B, wl.V), dtype=torch.bfloat16, device="cuda")
    return [lambda i: fs.sample_fused(Hb, Ws[i % len(Ws)], T, seed, i, out=out, workspace=ws),
            lambda i: fs.sample_fused(Hb, Ws[i % len(Ws)], T, seed, i, out=out, workspace=ws, logits=logits),
            lambda i: fs.sample_unfused(Hb, Ws[i % len(Ws)], T, seed, i, torch.bfloat16, out=out, workspace=uws)]


def time_graph(fs, Hb, Ws, wl, steps, B, reps=20):
    """Decode steps 0 .. n-1 (n = min(steps, 64), each with its own step value,
    so its own noise) captured once in a HIP graph and replayed: ms per step
    with no host launch cost. The replayed tokens of the first and last step
    are checked against eager calls."""
    import torch
    n = min(steps, 64)
    tiled = isinstance(Ws[0], fs.TiledWeights)
    ws = torch.empty(fs.workspace_bytes(B, wl.D, wl.V, Hb.dtype, tiled=tiled), dtype=torch.uint8, device="cuda")
    outs = torch.empty((n, B), dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    calls = lambda: [fs.sample_fused(Hb, Ws[i % len(Ws)], wl.temperature, wl.seed, i, out=outs[i],
                                     workspace=ws, stream=s) for i in range(n)]
    with torch.cuda.stream(s):
        calls()                          # warm the calls on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / (reps * n)
    for i in (0, n - 1):
        eager = fs.sample_fused(Hb, Ws[i % len(Ws)], wl.temperature, wl.seed, i)
        assert torch.equal(eager, outs[i]), f"graph replay differs from the eager call at step {i}"
    return ms, n


def time_vendor_gemm(Hb, Wr, steps, warmup):
    """ms per torch.matmul (hipBLASLt) H @ W^T into a bf16 logits buffer,
    alternating the W copies: the library GEMM alone, with no noise and no
    argmax. Context for the contraction's speed, not a sampler baseline."""
    import torch
    B, V = Hb.shape[0], Wr[0].shape[0]
    outs = [torch.empty(B, V, dtype=torch.bfloat16, device="cuda") for _ in Wr]
    for i in range(max(warmup, 10)):
        torch.matmul(Hb, Wr[i % len(Wr)].t(), out=outs[i % len(Wr)])
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        torch.matmul(Hb, Wr[i % len(Wr)].t(), out=outs[i % len(Wr)])
    t1.record()
    torch.cuda.synchronize()
    del outs
    return t0.elapsed_time(t1) / steps


def cpu_baseline(H, W, wl, B, budget_s=12.0):
    """Times the CPU oracle on whole decode steps of this workload (all B rows,
    full vocabulary) until about budget_s seconds of work are done."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    steps = 0
    t0 = time.perf_counter()
    while True:
        oracle.sample(H[:B], W, wl.temperature, wl.seed, steps)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 30:
            break
    # one step split into its two parts: the fp64 logits (BLAS) and the rest
    # (Philox, Gumbel, perturbed argmax; numpy on one thread)
    t1 = time.perf_counter()
    oracle.exact_logits(H[:B], W)
    gemm_s = time.perf_counter() - t1
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:  # pragma: no cover
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count()
    return {"value": B * steps / el, "unit": "samples/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{steps} full decode step(s) of the workload (B={B} rows x V={wl.V}), "
                      f"{el:.1f} s on the host, fp64 numpy/BLAS",
            "seconds_per_step": el / steps, "logits_seconds_per_step": gemm_s,
            "noise_and_argmax_seconds_per_step": max(el / steps - gemm_s, 0.0),
            "cpu_model": cpu_model, "cpu_count": os.cpu_count(), "affinity_cores": affinity,
            "blas_threads": int(threads)}


def traffic_record(kernel: str, workload: str, B: int):
    """HBM bytes per launch measured with rocprofv3 counters for these exact
    sources, if such a record is committed under profiles/."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    key = f"{kernel}/{workload}/B{B}"
    r = rec.get(key)
    if not r or r.get("source_hash") != source_hash():
        return None
    return r.get("bytes_per_launch")


def oracle_timings(wl, H, W):
    """The CPU oracle on one decode step of this workload at every B of its
    sweep with the host's BLAS threads, and on one thread at B = 1 for the two
    smallest heads: end to end (widening, fp64 logits, Philox, Gumbel, top-2),
    then the fp64 logits alone, so each entry also splits the step into the
    logits (BLAS) and the rest (noise and argmax, numpy). Returns a list of
    dicts."""
    import oracle
    from threadpoolctl import threadpool_limits
    cases = [(B, 0) for B in wl.batches]
    if wl.name in ("tiny_f32", "llama3_8b"):
        cases.append((1, 1))
    out = []
    for B, threads in cases:
        with threadpool_limits(limits=threads if threads else None):
            t0 = time.perf_counter()
            oracle.sample(H[:B], W, wl.temperature, wl.seed, 0)
            sec = time.perf_counter() - t0
            t1 = time.perf_counter()
            oracle.exact_logits(H[:B], W)
            gemm = time.perf_counter() - t1
        out.append({"workload": wl.name, "B": B, "seconds": round(sec, 3), "samples_per_s": round(B / sec, 2),
                    "logits_seconds": round(gemm, 3), "noise_and_argmax_seconds": round(max(sec - gemm, 0.0), 3),
                    "threads": threads or "blas default"})
        log(f"[bench] oracle {wl.name} B={B} ({out[-1]['threads']} threads): {sec:.2f} s "
            f"(logits {gemm:.2f} s)")
    return out


def sweep_workload(fs, wl, steps, repeats, warm_ms, vendor=True, cpu=None):
    """Compact sweep entries for every B of one workload: the fused call on
    the layout the headline uses (tiled for bf16 heads, row-major for fp32),
    its Stage-1 HBM and matrix-core fractions, and beside it the plain call on
    row-major W, single-pass (B <= 8), the unfused baseline (bf16 logits), the
    store-logits option (IO-model check) and, for bf16 heads, the library GEMM
    alone. Returns a list of dicts; with a list as `cpu`, the CPU oracle's
    timings of this workload are appended to it."""
    import torch
    from lm_head_gemm_amd import inputs
    t = time.perf_counter()
    H = inputs.make_hidden(wl)
    W = inputs.make_weights(wl)
    Hd = upload(H)
    Wr = [upload(W), upload(W)]
    if cpu is not None:
        cpu += oracle_timings(wl, H, W)
    del H, W
    tiled = wl.dtype == "bf16"
    Wt = [fs.TiledWeights(w) for w in Wr] if tiled else Wr
    torch.cuda.synchronize()
    log(f"[bench] sweep {wl.name}: inputs ready in {time.perf_counter() - t:.1f} s")
    esz = 2 if wl.dtype == "bf16" else 4
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    out = []
    for B in wl.batches:
        Hb = Hd[:B]
        ms, s1, _ = time_fused(fs, Hb, Wt, wl, steps, 0, B, min_warm_ms=warm_ms, repeats=repeats)
        nt = fs.num_vocab_tiles(B, wl.D, wl.V, Hb.dtype, tiled=tiled)
        byts = stage1_bytes(B, wl.D, wl.V, esz, nt)
        flops = 2 * B * wl.V * wl.D
        e = {"workload": wl.name, "B": B, "us": ms * 1e3, "samples_per_s": B / (ms * 1e-3),
             "stage1_us": s1 * 1e3, "hbm_frac": byts / (s1 * 1e-3) / 1e9 / HBM_PEAK_GBS,
             "mfma_frac": flops / (s1 * 1e-3) / 1e12 / mfma_peak,
             "layout": "tiled" if tiled else "rows"}
        if tiled:
            rms, _, _ = time_fused(fs, Hb, Wr, wl, steps, 0, B, min_warm_ms=warm_ms, repeats=repeats)
            e["rows_us"] = rms * 1e3
        if B <= 8:
            sms, _, _ = time_fused(fs, Hb, Wt, wl, steps, 0, B, single_pass=True, min_warm_ms=warm_ms,
                                   repeats=repeats)
            e["single_pass_us"] = sms * 1e3
        # the IO-model check: plain, store-logits and unfused calls timed in
        # alternating runs (like with like)
        pl, st, u16 = time_interleaved(io_model_calls(fs, Hb, Wt, wl, B), steps, repeats, warm_ms)
        e.update({"unfused_us": u16 * 1e3, "fused_speedup": u16 / ms,
                  "store_overhead": st / pl - 1.0, "store_overhead_io_model": B / wl.D,
                  "unfused_overhead": u16 / pl - 1.0, "unfused_overhead_io_model": 2 * B / wl.D})
        if vendor and tiled:
            e["vendor_gemm_us"] = time_vendor_gemm(Hb, Wr, steps, 10) * 1e3
        log(f"[bench] sweep {wl.name} B={B}: {e['us']:.1f} us (stage1 {e['stage1_us']:.1f}, "
            f"HBM {e['hbm_frac']:.2f}, MFMA {e['mfma_frac']:.2f}), unfused {e['unfused_us']:.1f}"
            + (f", rows {e['rows_us']:.1f}" if "rows_us" in e else ""))
        out.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in e.items()})
    del Hd, Wr, Wt
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed runs of --steps calls for the headline; value is from the median run")
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--batch", type=int, default=0,
                    help="batch rows per step (default: 64, or the largest of the workload's sweep below 64)")
    ap.add_argument("--sweep", action="store_true",
                    help="also time every B of the headline workload's sweep with the headline's full detail")
    ap.add_argument("--no-all-sweep", action="store_true",
                    help="skip the compact sweep over every workload and every B of its sweep")
    ap.add_argument("--sweep-steps", type=int, default=20, help="calls per timed run in the compact sweep")
    ap.add_argument("--sweep-repeats", type=int, default=3, help="timed runs per point in the compact sweep")
    ap.add_argument("--sweep-workloads", default="tiny_f32,llama3_8b,qwen_7b,llama3_70b,deepseek_v3")
    ap.add_argument("--batches", default="", help="comma-separated batch sizes to sweep instead")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unfused", action="store_true")
    ap.add_argument("--variant", default="auto", choices=["auto", "gemv", "mfma"])
    ap.add_argument("--vocab-tile", type=int, default=0)
    ap.add_argument("--batch-tile", type=int, default=0)
    ap.add_argument("--temperature", type=float, default=None,
                    help="override the workload's temperature (0 = greedy, no noise)")
    ap.add_argument("--layout", default="auto", choices=["auto", "rows", "tiled"],
                    help="W row-major, or repacked once into the tiled matrix-core layout "
                         "(auto: tiled for bf16 heads, row-major for fp32 ones; the tiled layout is bf16 only)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run only a device copy of this size (counter calibration) and exit")
    ap.add_argument("--probe", action="store_true",
                    help="also stream W once per step with the read probe (attainable bandwidth)")
    ap.add_argument("--no-rows", action="store_true", help="skip timing the row-major layout beside")
    ap.add_argument("--graph", action="store_true",
                    help="also time the decode steps captured in one HIP graph and replayed (no host launch cost)")
    ap.add_argument("--no-vendor", action="store_true",
                    help="skip timing the library GEMM (torch.matmul, logits only) beside, for context")
    ap.add_argument("--group-size", type=int, default=16384,
                    help="also time the grouped variant with groups of this many vocab entries (0: skip)")
    ap.add_argument("--single-pass", action="store_true",
                    help="time the one-launch form (Stage 2 folded into Stage 1) as the headline")
    ap.add_argument("--min-warmup-ms", type=float, default=300.0,
                    help="keep warming up (untimed) until this much wall time has passed")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the whole vocabulary "
              f"fits one MI355X; the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    from lm_head_gemm_amd import flashsample as fs
    from lm_head_gemm_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 10}))
        return

    wl = inputs.WORKLOADS[args.workload]
    if args.layout == "auto":
        args.layout = "tiled" if wl.dtype == "bf16" else "rows"
    if args.temperature is not None:
        import dataclasses
        wl = dataclasses.replace(wl, temperature=args.temperature)
    B = args.batch or max(b for b in wl.batches if b <= 64)
    log(f"[bench] generating {wl.name}: D={wl.D} V={wl.V} {wl.dtype}, B={B}")
    t = time.perf_counter()
    b_need = max([wl.b_max, B] + [int(x) for x in args.batches.split(",") if x])
    H = inputs.make_hidden(wl, b_max=b_need)
    W = inputs.make_weights(wl)
    log(f"[bench] inputs ready in {time.perf_counter() - t:.1f} s; uploading")
    Hd = upload(H)
    # two resident copies of W, alternated, so no step can reuse the previous
    # step's tail of W from the 256 MB last-level cache
    Ws = [upload(W), upload(W)]
    esz = 2 if wl.dtype == "bf16" else 4
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS

    single = args.single_pass

    def run(b, weights=None, single_pass=None):
        main_weights = weights is None
        weights = Ws if weights is None else weights
        single_pass = single if single_pass is None else single_pass
        Hb = Hd[:b]
        runs = []
        ms, s1, n_warm = time_fused(fs, Hb, weights, wl, args.steps, args.warmup, b, args.variant,
                                    args.vocab_tile, args.batch_tile, single_pass, args.min_warmup_ms,
                                    repeats=args.repeats, runs_out=runs)
        tiled = isinstance(weights[0], fs.TiledWeights)
        nt = fs.num_vocab_tiles(b, wl.D, wl.V, Hb.dtype, args.variant, args.vocab_tile, tiled=tiled)
        byts = stage1_bytes(b, wl.D, wl.V, esz, nt)
        flops = 2 * b * wl.V * wl.D
        rec = {"B": b, "ms_per_step": ms, "samples_per_s": b / (ms * 1e-3), "stage1_ms": s1,
               "stage1_GBps": byts / (s1 * 1e-3) / 1e9, "stage1_bytes": byts, "n_tiles": nt,
               "hbm_frac": byts / (s1 * 1e-3) / 1e9 / HBM_PEAK_GBS,
               "flops": flops, "stage1_TFLOPs": flops / (s1 * 1e-3) / 1e12,
               "mfma_frac": flops / (s1 * 1e-3) / 1e12 / mfma_peak,
               "warmup_steps_run": n_warm, "ms_per_step_runs": runs, "ms_per_step_min": min(runs)}
        if not args.no_unfused:
            u16 = time_unfused(fs, Hb, weights, wl, args.steps, args.warmup, b, torch.bfloat16,
                               args.min_warmup_ms)
            rec["unfused_bf16_ms_per_step"] = u16
            rec["fused_speedup_vs_unfused_bf16"] = u16 / ms
            u32 = time_unfused(fs, Hb, weights, wl, args.steps, args.warmup, b, torch.float32,
                               args.min_warmup_ms)
            rec["unfused_f32_ms_per_step"] = u32
            rec["fused_speedup_vs_unfused_f32"] = u32 / ms
            # IO model (Section 3): with bf16 logits, the unfused path moves
            # 2*B*V*2 bytes more than the fused one (write + read back) and the
            # store-logits option B*V*2 more (write), on top of the V*D*2 of W.
            # The three calls are timed in alternating runs for this comparison.
            pl, st, ui = time_interleaved(io_model_calls(fs, Hb, weights, wl, b), args.steps, args.repeats,
                                          args.min_warmup_ms)
            rec["io_model"] = {"timing": "plain, store-logits and unfused calls in alternating runs",
                               "plain_ms_per_step": pl, "store_logits_ms_per_step": st,
                               "unfused_ms_per_step": ui,
                               "store_overhead": st / pl - 1.0,
                               "store_overhead_predicted": b / wl.D,
                               "unfused_overhead": ui / pl - 1.0,
                               "unfused_overhead_predicted": 2 * b / wl.D,
                               "unfused_f32_overhead": u32 / ms - 1.0,
                               "unfused_f32_overhead_predicted": 2 * b * 4 / (wl.D * esz)}
        if main_weights and vendor_rows is not None and wl.dtype == "bf16":
            vg = time_vendor_gemm(Hb, vendor_rows, args.steps, args.warmup)
            rec["vendor_gemm_logits_only_ms"] = vg
            rec["fused_vs_vendor_gemm_only"] = vg / ms
        log(f"[bench] B={b}: {ms * 1e3:.1f} us/step, stage1 {s1 * 1e3:.1f} us "
            f"({rec['stage1_GBps']:.0f} GB/s, {rec['stage1_TFLOPs']:.0f} TFLOP/s)" +
            (f", unfused {rec['unfused_bf16_ms_per_step'] * 1e3:.1f} us, store-logits overhead "
             f"{rec['io_model']['store_overhead'] * 100:+.1f}% (IO model {b / wl.D * 100:+.1f}%)"
             if not args.no_unfused else ""))
        return rec

    Ws_rows = Ws
    vendor_rows = None if args.no_vendor else Ws_rows
    if args.layout == "tiled":
        Ws = [fs.TiledWeights(w) for w in Ws_rows]
        torch.cuda.synchronize()
        if args.no_rows:
            del Ws_rows
            Ws_rows = None
            if vendor_rows is None:
                torch.cuda.empty_cache()

    head = run(B)
    sweep_bs = [int(x) for x in args.batches.split(",") if x] or (list(wl.batches) if args.sweep else [])
    sweep = [run(b) for b in sweep_bs if b != B]

    torch.cuda.synchronize()
    result = {
        "metric": "samples/s, fused LM-head sampler (Gumbel-max), V=128256 D=4096",
        "value": head["samples_per_s"],
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": head["warmup_steps_run"],
        "ms_per_step": head["ms_per_step"],
        "repeats": args.repeats,
        "ms_per_step_runs": head["ms_per_step_runs"],
        "ms_per_step_min": head["ms_per_step_min"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded Gaussian head, FS-DATA-1)",
        "config": {"workload": wl.name, "B": B, "D": wl.D, "V": wl.V, "temperature": wl.temperature,
                   "weights_layout": args.layout, "stage2": "folded into stage 1" if single else "separate kernel",
                   "vocab_tiles": head["n_tiles"], "W_copies_alternated": 2},
        "roofline": roofline(head, mfma_peak, traffic_record("stage1", wl.name, B)),
    }
    other = run(B, single_pass=not single)
    result["single_pass" if not single else "two_stage"] = {
        "ms_per_step": other["ms_per_step"], "samples_per_s": other["samples_per_s"],
        "stage1_us": other["stage1_ms"] * 1e3}
    if args.layout == "tiled" and args.group_size > 0:
        # the grouped variant (local sample + log-mass per group, group drawn
        # from the log-masses), groups shaped like vocabulary shards
        gms, gs1, _ = time_fused(fs, Hd[:B], Ws, wl, args.steps, args.warmup, B, single_pass=False,
                                 min_warm_ms=args.min_warmup_ms, group_size=args.group_size)
        result["grouped"] = {"group_size": args.group_size, "n_groups": -(-wl.V // args.group_size),
                             "ms_per_step": gms, "samples_per_s": B / (gms * 1e-3), "stage1_us": gs1 * 1e3,
                             "overhead_vs_plain": gms / head["ms_per_step"] - 1.0}
        log(f"[bench] grouped (G={args.group_size}): {gms * 1e3:.1f} us/step, stage1 {gs1 * 1e3:.1f} us")
    if args.layout == "tiled" and Ws_rows is not None:
        rows = run(B, Ws_rows, single_pass=False)
        result["rows_layout"] = {"ms_per_step": rows["ms_per_step"], "samples_per_s": rows["samples_per_s"],
                                 "stage1_us": rows["stage1_ms"] * 1e3, "stage1_GBps": rows["stage1_GBps"]}
    if args.probe:
        if Ws_rows is not None:
            src = Ws_rows[0]
        else:
            src = Ws[0].data if isinstance(Ws[0], fs.TiledWeights) else Ws[0]
        flat = src.reshape(-1)
        sink = fs.probe_read(flat)
        for _ in range(5):
            fs.probe_read(flat, sink=sink)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(args.steps):
            fs.probe_read(flat, sink=sink)
        t1.record()
        torch.cuda.synchronize()
        pms = t0.elapsed_time(t1) / args.steps
        nbytes = flat.numel() * flat.element_size()
        result["read_probe"] = {"bytes": nbytes, "us": pms * 1e3, "GBps": nbytes / (pms * 1e-3) / 1e9}
    if args.graph:
        gms, gn = time_graph(fs, Hd[:B], Ws, wl, args.steps, B)
        result["graph_replay"] = {"steps_per_graph": gn, "ms_per_step": gms, "samples_per_s": B / (gms * 1e-3),
                                  "speedup_over_launched": head["ms_per_step"] / gms}
        log(f"[bench] graph replay: {gms * 1e3:.1f} us/step over {gn} captured steps")
    if "vendor_gemm_logits_only_ms" in head:
        result["vendor_gemm_context"] = {
            "what": "torch.matmul (hipBLASLt) H @ W^T -> bf16 logits only: no noise, no argmax, not a sampler",
            "ms": head["vendor_gemm_logits_only_ms"],
            "fused_call_speedup_over_it": head["fused_vs_vendor_gemm_only"]}
    if "unfused_bf16_ms_per_step" in head:
        result["unfused_bf16"] = {"ms_per_step": head["unfused_bf16_ms_per_step"],
                                  "samples_per_s": B / (head["unfused_bf16_ms_per_step"] * 1e-3),
                                  "fused_speedup": head["fused_speedup_vs_unfused_bf16"]}
        result["unfused_f32"] = {"ms_per_step": head["unfused_f32_ms_per_step"],
                                 "samples_per_s": B / (head["unfused_f32_ms_per_step"] * 1e-3),
                                 "fused_speedup": head["fused_speedup_vs_unfused_f32"]}
        result["io_model"] = head["io_model"]
    if sweep:
        result["sweep_headline_workload"] = [head] + sweep
    if not args.no_all_sweep:
        # free the headline's buffers first: the sweep holds two copies of each head
        del Hd, Ws
        Ws_rows = vendor_rows = None
        torch.cuda.empty_cache()
        entries = []
        cpu = None if args.no_cpu_baseline else []
        for name in [x for x in args.sweep_workloads.split(",") if x]:
            entries += sweep_workload(fs, inputs.WORKLOADS[name], args.sweep_steps, args.sweep_repeats,
                                      min(args.min_warmup_ms, 100.0), vendor=not args.no_vendor, cpu=cpu)
        result["sweep"] = {"steps": args.sweep_steps, "repeats": args.sweep_repeats,
                           "layout": "tiled for bf16 heads, row-major for fp32", "entries": entries}
        if cpu:
            result["sweep"]["oracle_cpu"] = cpu
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(H, W, wl, B)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
