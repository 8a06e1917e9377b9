#!/usr/bin/env python3
"""PISA prefill benchmark on one MI355X (gfx950).

One step = one pass of the whole hot path over one batch of synthetic input
already resident in HBM: key pyramid (pisa_build_pyramid), two-stage
selection (pisa_select) and block-sparse attention (pisa_sparse_attn).
Default workload: prefill N=131072, B=1, Hq=32, Hkv=8, d=128, C=64, g=2,
K=16, bf16, causal, planted needle leaves.  Prints ONE JSON line.

Also measured in the same process: the flat single-level selector on the same
inputs (leaf pooling + flat top-K), per-kernel times from HIP events recorded
on the launch stream (library timer), the roofline of the dominant kernel and
of the others (stage-1 routing against the on-chip gather rate measured by
the library's gather probe), and the CPU oracle timed on a bounded sample of
query positions (with a parity summary of the GPU outputs at those
positions).  The default 128K run then runs the metric's other sequence
length, N=262144 (C=128, K=32, shared needle spans), in the same process and
adds it to the line as "prefill_256k" (step, select and flat-select times,
its dominant kernel's roofline, a sampled parity summary), then the fused
decode step over 64 sequences of 131072 cached tokens (all 256 of its decode
steps timed) as "decode_128k".
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = {"hbm_GBps": 8000.0, "mfma_bf16_TFLOPs": 2500.0, "mfma_f32_TFLOPs": 157.3}
METRIC = "PISA select+sparse-attn prefill tokens/s and select ms at 128K/256K, 1 GPU"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="prefill_128k")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target wall time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flat", action="store_true")
    ap.add_argument("--no-256k", action="store_true",
                    help="skip the 256K sub-leg that the default 128K run adds to its JSON line")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the fused decode leg the default 128K run adds to the line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy first (reference for HBM counter scaling)")
    ap.add_argument("--scaling", action="store_true",
                    help="selection-time scaling and PISA-vs-flat crossover at C=64, K=16 over --scaling-n")
    ap.add_argument("--scaling-n", default="32768,65536,131072,262144,524288,1048576")
    ap.add_argument("--scaling-positions", type=int, default=48,
                    help="query positions per N checked against the oracle in the scaling leg")
    ap.add_argument("--backward", action="store_true",
                    help="sparse-attention forward + backward over the workload's selection")
    ap.add_argument("--io", action="store_true",
                    help="one-stage vs two-stage selection at G_Q = 4 and 16 (N = 131072, C = 64, K = 16)")
    return ap.parse_args()


def dev(x):
    import numpy as np
    import torch

    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def source_digest() -> str:
    """Digest of the HIP sources: counter summaries taken from other sources
    are stale."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "hierarchical_block_sparse_mean_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(fn.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from profiles/traffic_<kernel>_<workload>.txt
    (rocprofv3 FETCH_SIZE / WRITE_SIZE scaled by a 1 GiB copy), or None if
    absent or taken from other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                vals[key.strip()] = val.strip()
    if vals.get("source_digest") != source_digest():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def measured_ceilings() -> dict:
    """Ceilings measured on this GPU, next to the vendor peaks: a 1 GiB
    device-to-device copy by the platform (2 GiB of HBM traffic per copy), the
    library's 16-byte streaming probe reading 2 GiB and copying 1 GiB (best of
    a few grid sizes), and a bf16 GEMM (8192^3, the platform BLAS), each timed
    with HIP events.  The HBM ceiling the memory-bound kernels are compared
    with (`hbm_GBps`) is the best of the three streams: mostly-read kernels
    exceed a copy's rate."""
    import torch

    from hierarchical_block_sparse_mean_amd import pisa

    src = torch.empty(1 << 30, dtype=torch.int16, device="cuda")
    src.fill_(1)
    dst = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
    a = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")
    wgs = 256 * 16
    sink = torch.empty(wgs * 256, dtype=torch.int32, device="cuda")
    half = src[: 1 << 29]

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1000.0

    copy_s = timed(lambda: dst.copy_(half), 10)
    read_s = min(timed(lambda: pisa.probe_stream(src, None, 2 << 30, 0, n, sink), 10) for n in (256, 512, 1024, wgs))
    pcopy_s = min(timed(lambda: pisa.probe_stream(half, dst, 1 << 30, 1, n, None), 10) for n in (256, 1024, wgs))
    gemm_s = timed(lambda: torch.matmul(a, b), 10)
    del src, dst, a, b, sink, half
    torch.cuda.empty_cache()
    out = {"copy_GBps": round(2 * (1 << 30) / copy_s / 1e9, 1),
           "stream_read_GBps": round(2 * (1 << 30) / read_s / 1e9, 1),
           "stream_copy_GBps": round(2 * (1 << 30) / pcopy_s / 1e9, 1),
           "gemm_bf16_TFLOPs": round(2 * 8192 ** 3 / gemm_s / 1e12, 1)}
    out["hbm_GBps"] = max(out["copy_GBps"], out["stream_read_GBps"], out["stream_copy_GBps"])
    return out


def attended_keys(idx, N: int, C: int, causal: bool):
    """Sum over (b, h, t, slot) of the keys attention reads for that leaf."""
    import torch

    j = idx.long()
    t = torch.arange(N, device=idx.device).view(1, 1, N, 1)
    lo = j * C
    hi = torch.clamp(lo + C, max=N)
    if causal:
        hi = torch.minimum(hi, t + 1)
    keys = torch.where(j >= 0, torch.clamp(hi - lo, min=0), torch.zeros_like(j))
    return int(keys.sum().item())


def attention_pairs(N: int, C: int, D: int, dtype: str) -> bool:
    """Whether the library attends kept sibling pairs as one tile: C <= 64
    (fp32 only with d = 64) or C <= 128 for bf16, unless the level-2 blocks
    would push a head's clustering off its 16384-bin LDS histogram while the
    leaves alone fit it."""
    M1 = -(-N // C)
    M2 = -(-M1 // 2)
    fits = (dtype == "bf16" or D <= 64) if C <= 64 else dtype == "bf16"
    return fits and (M1 + M2 <= 16384 or M1 > 16384)


def attention_partials(idx, paired: bool) -> int:
    """Partial (query, slot) records the attention writes and the merge reads
    per KV head: one per kept leaf, except that with sibling pairing a leaf
    kept together with its sibling (even j followed by j + 1 in the ascending
    row) shares one record with it."""
    j = idx.long()
    kept = int((j >= 0).sum().item())
    if not paired:
        return kept
    both = (j[..., :-1] >= 0) & (j[..., :-1] % 2 == 0) & (j[..., 1:] == j[..., :-1] + 1)
    return kept - int(both.sum().item())


def stage1_scored_keys(blk2, N: int, C: int, causal: bool):
    """Keys scored by stage 2: both leaves of every kept level-2 block."""
    import torch

    j2 = blk2.long()
    t = torch.arange(N, device=blk2.device).view(1, 1, N, 1)
    total = 0
    pairs = int((j2 >= 0).sum().item())
    for l in (0, 1):
        lo = (2 * j2 + l) * C
        hi = torch.clamp(lo + C, max=N)
        if causal:
            hi = torch.minimum(hi, t + 1)
        total += int(torch.where(j2 >= 0, torch.clamp(hi - lo, min=0), torch.zeros_like(j2)).sum().item())
    return total, pairs


def l2_gather_ceiling(D: int, rows_per_head: int, heads: int) -> dict:
    """On-chip gather ceiling of stage-1 routing: the library's gather probe
    (tiles of 16 fp16 rows at pseudo-random rows of a table sized like the
    summary levels stage 1 reads from memory, loaded and transposed through
    LDS as stage 1 does, one persistent workgroup of 16 waves per compute
    unit) timed with HIP events.  Returns the rate in GB/s."""
    import torch

    from hierarchical_block_sparse_mean_amd import pisa

    wgs = 256
    table = torch.randn(heads * rows_per_head * D, device="cuda").to(torch.float16)
    sink = torch.empty(wgs * 16 * 64, dtype=torch.int32, device="cuda")
    tiles = 1024
    pisa.probe_gather(table, rows_per_head, heads, D, wgs, tiles, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        pisa.probe_gather(table, rows_per_head, heads, D, wgs, tiles, sink)
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) / reps / 1000.0
    nbytes = wgs * 16 * tiles * 16 * D * 2
    return {"GBps": round(nbytes / s / 1e9, 1), "bytes_per_launch": nbytes, "rows_per_head": rows_per_head,
            "heads": heads, "note": "random 16-row fp16 tiles from an L2-resident table per head, 16 waves per CU, "
                                    "128-byte row pieces per eight lanes through an LDS tile into the MFMA operand "
                                    "layout (stage 1's access pattern), no other work"}


def stage_levels_in_memory(N: int, C: int, D: int) -> int:
    """Summary rows per head of the levels stage 1 reads from memory (those
    below its LDS stage: the stage holds every level whose rows, with the
    levels above it, fit what 16 waves' candidate lists and gather tiles leave
    of 160 KB, at (D + 8) * 2 + 4 bytes per row)."""
    from hierarchical_block_sparse_mean_amd import pisa

    L = pisa.levels(N, C)
    M = [pisa.level_rows(N, C, l) for l in range(1, L + 1)]
    pitch = (D + 8) * 2 + 4
    budget = 160 * 1024 - 16 * (1024 + 16 * (D + 8) * 2)
    for l in range(1, L + 1):
        if sum(M[l - 1:]) * pitch <= budget:
            return sum(M[: l - 1])
    return sum(M)


def flat_work(N: int, C: int, D: int, B: int, Hkv: int, causal: bool) -> float:
    """Flops of the flat selector in its summed-query form: 2 d per (b, h, t,
    valid leaf)."""
    import numpy as np

    M1 = -(-N // C)
    t = np.arange(N, dtype=np.int64)
    valid = np.minimum(M1, t // C + 1) if causal else np.full(N, M1)
    return 2.0 * D * float(valid.sum()) * B * Hkv


def prefill_leg(args, w, ceilings, steps: int, warmup: int, cpu_leg: bool, parity_positions: int | None) -> dict:
    """One prefill workload: K timed steps (pyramid + two-stage select +
    attention), per-kernel times from a second pass, rooflines, the flat
    selector, and (cpu_leg) the oracle on a bounded sample or (parity_positions)
    a sampled parity summary."""
    import numpy as np
    import torch

    from hierarchical_block_sparse_mean_amd import inputs as I
    from hierarchical_block_sparse_mean_amd import pisa

    log(f"workload {w.name}: B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} D={w.D} C={w.C} K={w.K} {w.dtype} "
        f"causal={w.causal} needles={w.needles}")
    t0 = time.perf_counter()
    data = I.generate(w)
    log(f"inputs generated in {time.perf_counter() - t0:.1f}s")
    q, k, v = dev(data["q"]), dev(data["k"]), dev(data["v"])
    p = pisa.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=w.causal, dtype=w.dtype)
    pyr = pisa.alloc_pyramid(p)
    ws = pisa.workspace(pisa.select_workspace_bytes(p))
    idx = torch.empty((w.B, w.Hkv, w.N, w.K), dtype=torch.int32, device="cuda")
    score = torch.empty_like(idx, dtype=torch.float32)
    o = torch.empty_like(q)
    attn_ws = pisa.workspace(pisa.attn_workspace_bytes(p))

    def step(ev=None):
        if ev:
            ev[0].record()
        pisa.build_pyramid(p, k, pyr)
        if ev:
            ev[1].record()
        pisa.select(p, q, k, pyr, idx=idx, score=score, ws=ws)
        if ev:
            ev[2].record()
        pisa.sparse_attn(p, q, k, v, idx, o=o, lse=None, ws=attn_ws, with_lse=False)
        if ev:
            ev[3].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {warmup} steps done")

    # timed region: the K steps with four stage events each; the library's
    # per-launch events (about 1% of a step) are recorded in a second pass of
    # K steps on the same inputs, for the per-kernel times
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    pisa.timer_enable(True)
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    kernels = pisa.timer_report()
    pisa.timer_enable(False)
    stage = {"pyramid": 0.0, "select": 0.0, "attention": 0.0}
    for e in evs:
        stage["pyramid"] += e[0].elapsed_time(e[1])
        stage["select"] += e[1].elapsed_time(e[2])
        stage["attention"] += e[2].elapsed_time(e[3])
    stage = {kk: vv / steps for kk, vv in stage.items()}
    ms_per_step = wall * 1000.0 / steps
    value = w.B * w.N / (ms_per_step / 1000.0)
    log(f"timed {steps} steps: {ms_per_step:.3f} ms/step, stages {stage}")
    per_kernel = {name: {"launches": n, "avg_ms": tot / n, "ms_per_step": tot / steps}
                  for name, (n, tot) in kernels.items()}

    # ---- algorithmic work of the kernels (per step) ----------------------------
    G = w.gq
    esize = 2 if w.dtype == "bf16" else 4
    mfma_peak = PEAK["mfma_bf16_TFLOPs"] if w.dtype == "bf16" else PEAK["mfma_f32_TFLOPs"]
    blk2 = pisa.select_level2(p, ws)
    scored_keys, s1_pairs = stage1_scored_keys(blk2, w.N, w.C, w.causal)
    attn_keys = attended_keys(idx, w.N, w.C, w.causal)
    partials = attention_partials(idx, attention_pairs(w.N, w.C, w.D, w.dtype))
    M = [pisa.level_rows(w.N, w.C, l) for l in range(1, pisa.levels(w.N, w.C) + 1)]
    rc = pisa.route_counts(p, q, k, pyr) if w.dtype == "bf16" else None
    work = {
        # 4 d flops per attended (query head, key): q.k and p.v
        "attn_leaf": ("mfma", 4.0 * w.D * G * attn_keys, "TFLOP/s",
                      f"4*d flop per attended (query head, key); {attn_keys * G} such pairs"),
        "attn_query": ("mfma", 4.0 * w.D * G * attn_keys, "TFLOP/s",
                       f"4*d flop per attended (query head, key); {attn_keys * G} such pairs"),
        # 2 d flops per scored (query head, raw key)
        "leaf_score": ("mfma", 2.0 * w.D * G * scored_keys, "TFLOP/s",
                       f"2*d flop per scored (query head, raw key); {scored_keys * G} such pairs from {s1_pairs} "
                       "(query, kept level-2 block) pairs"),
        # read every key once, write leaf means and the four levels above them
        "pyr_leaf": ("hbm", float(w.B * w.Hkv * (w.N * w.D * esize + sum(M[:5]) * w.D * 4)), "GB/s",
                     "N*d*elem read + (M1+..+M5)*d*4 written per (b, h)"),
        # merge: read G partial rows (d elems + m, l) per partial record, write o
        "attn_merge": ("hbm", float(partials * G * (w.D * esize + 8) + w.B * w.Hq * w.N * w.D * esize), "GB/s",
                       f"per partial record (query, kept leaf or kept sibling pair; {partials} records): "
                       "G*(d*elem + 8) bytes read; o written once"),
    }

    def rate(name, amount, unit):
        launches = per_kernel[name]["launches"] / steps
        avg_s = per_kernel[name]["avg_ms"] / 1000.0
        per_launch = amount / launches
        return per_launch, avg_s, per_launch / avg_s / (1e12 if unit == "TFLOP/s" else 1e9)

    dominant = max(per_kernel, key=lambda n: per_kernel[n]["ms_per_step"])
    roofline = None
    if dominant in work:
        bound, amount, unit, note = work[dominant]
        per_launch, avg_s, achieved = rate(dominant, amount, unit)
        peak = mfma_peak if unit == "TFLOP/s" else PEAK["hbm_GBps"]
        measured = ceilings["hbm_GBps"] if unit == "GB/s" else ceilings["gemm_bf16_TFLOPs"]
        roofline = {"kernel": dominant, "bound": bound, "achieved": round(achieved, 3), "peak": peak,
                    "unit": unit, "frac": round(achieved / peak, 5),
                    "measured_peak": measured, "frac_of_measured": round(achieved / measured, 5),
                    "traffic": traffic_for(dominant, w.name),
                    "avg_launch_ms": round(per_kernel[dominant]["avg_ms"], 4),
                    "work_per_launch": per_launch, "work_note": note}
        if roofline["traffic"]:
            # the measured HBM bytes per launch as a rate, next to the copy
            # ceiling: how close the kernel's own data movement is to HBM
            tr = roofline["traffic"] / avg_s / 1e9
            roofline["traffic_GBps"] = round(tr, 1)
            roofline["traffic_frac_of_measured_hbm"] = round(tr / ceilings["hbm_GBps"], 4)
    kernel_rooflines = {}
    for name, (bound, amount, unit, note) in work.items():
        if name not in per_kernel:
            continue
        _, _, ach = rate(name, amount, unit)
        if unit == "TFLOP/s":
            kernel_rooflines[name] = {"bound": bound, "achieved_TFLOPs": round(ach, 2),
                                      "frac": round(ach / mfma_peak, 4),
                                      "frac_of_measured": round(ach / ceilings["gemm_bf16_TFLOPs"], 4)}
        else:
            kernel_rooflines[name] = {"bound": bound, "achieved_GBps": round(ach, 1),
                                      "frac": round(ach / PEAK["hbm_GBps"], 4),
                                      "frac_of_measured": round(ach / ceilings["hbm_GBps"], 4)}
    if rc is not None and "route_stage1" in per_kernel:
        # stage 1 reads its child summaries as fp16 rows (d*2 bytes); the
        # coarse levels come from LDS, the finer ones are gathered from memory
        # (L2-resident per head).  Bound: the on-chip gather rate of those
        # rows, measured by the gather probe on a table of the same size.
        rows_mem = rc["child_rows_from_memory"]
        ceil = l2_gather_ceiling(w.D, stage_levels_in_memory(w.N, w.C, w.D), w.B * w.Hkv)
        avg_s = per_kernel["route_stage1"]["avg_ms"] / 1000.0
        launches = per_kernel["route_stage1"]["launches"] / steps
        ach = rows_mem * w.D * 2 / launches / avg_s / 1e9
        kernel_rooflines["route_stage1"] = {
            "bound": "l2_gather", "achieved_GBps": round(ach, 1), "peak_GBps": ceil["GBps"],
            "peak_kind": "measured gather probe (on-chip, no published figure)", "frac": round(ach / ceil["GBps"], 4),
            "rows_from_memory": rows_mem, "rows_from_lds": rc["child_rows"] - rows_mem,
            "note": f"{rows_mem} child rows x d*2 B gathered from memory per launch over the launch time; "
                    f"{rc['child_rows'] - rows_mem} more rows come from the coarse levels staged in LDS; "
                    f"{rc['child_rows'] / max(1, rc['queries']):.1f} rows and "
                    f"{rc['scored_levels'] / max(1, rc['queries']):.2f} scored levels per (t, h)",
            "probe": ceil}

    # ---- flat single-level selector on the same inputs ------------------------
    flat_ms = None
    if not args.no_flat:
        fidx = torch.empty_like(idx)
        for _ in range(max(1, warmup)):
            pisa.build_pyramid(p, k, pyr)
            pisa.flat_select(p, q, pyr, idx=fidx, with_score=False)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            pisa.build_pyramid(p, k, pyr)
            pisa.flat_select(p, q, pyr, idx=fidx, with_score=False)
        e1.record()
        torch.cuda.synchronize()
        flat_ms = e0.elapsed_time(e1) / steps
        pisa.timer_enable(True)
        for _ in range(steps):
            pisa.flat_select(p, q, pyr, idx=fidx, with_score=False)
        torch.cuda.synchronize()
        fk = pisa.timer_report()
        pisa.timer_enable(False)
        if "flat" in fk:
            n_f, tot_f = fk["flat"]
            avg_s = tot_f / n_f / 1000.0
            ach = flat_work(w.N, w.C, w.D, w.B, w.Hkv, w.causal) / avg_s / 1e12
            kernel_rooflines["flat"] = {
                "bound": "mfma", "achieved_TFLOPs": round(ach, 2), "frac": round(ach / mfma_peak, 4),
                "frac_of_measured": round(ach / ceilings["gemm_bf16_TFLOPs"], 4), "avg_launch_ms": round(avg_s * 1e3, 4),
                "note": "2*d flop per (t, KV head, valid leaf): one logit per leaf summary with the group's "
                        "queries summed first; the kernel also keeps a top-K per query"}
        log(f"flat selector (leaf pooling + flat top-K): {flat_ms:.3f} ms")
        # re-run the PISA step so idx/score/o hold its outputs for the parity summary
        step()
        torch.cuda.synchronize()

    # ---- CPU oracle on a bounded sample, or a sampled parity summary -------------
    cpu = None
    parity = None
    if cpu_leg or parity_positions:
        import oracle

        op = oracle.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=w.causal)
        rng = np.random.default_rng(w.seed + 99)

        def sample(n):
            base = np.linspace(0, w.N, n, endpoint=False)
            return np.unique(np.minimum(w.N - 1, (base + rng.uniform(0, w.N / n)).astype(np.int64)))

        if cpu_leg:
            # calibrate the per-position cost (two sizes, so the per-head pyramid
            # build cancels), then size the sample to about cpu_seconds of wall time
            def timed(n):
                tt = sample(n)
                ta = time.perf_counter()
                ii, _, _, _ = oracle.select(op, data["q"], data["k"], ts=tt)
                oracle.attention(op, data["q"], data["k"], data["v"], ii, ts=tt)
                return time.perf_counter() - ta

            t_small, t_big = timed(64), timed(512)
            per_pos = max((t_big - t_small) / 448.0, 1e-5)
            fixed = max(t_small - 64 * per_pos, 0.0)
            n_main = int(min(16384, max(256, (args.cpu_seconds - fixed) / per_pos)))
            log(f"oracle sample: {n_main} positions (calibration: {per_pos * 1e3:.2f} ms/position, {fixed:.2f}s fixed)")
        else:
            n_main = parity_positions
        ts = sample(n_main)
        t_a = time.perf_counter()
        o_idx, o_score, o_gap, cnt = oracle.select(op, data["q"], data["k"], ts=ts)
        o_o, _ = oracle.attention(op, data["q"], data["k"], data["v"], o_idx, ts=ts)
        t_cpu = time.perf_counter() - t_a
        if cpu_leg:
            cpu = {"value": round(len(ts) / t_cpu, 3), "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
                   "sample": f"{len(ts)} query positions spread evenly over t in [0, {w.N}), every (b, KV head); "
                             f"oracle pyramid per head + selection + attention, fp64, {t_cpu:.1f}s wall"}
        g_idx = idx.cpu().numpy()[:, :, ts]
        g_score = score.cpu().numpy()[:, :, ts].astype(np.float64)
        same = (g_idx == o_idx).all(-1)
        exempt = o_gap < 1e-3
        m = same[..., None] & (o_idx >= 0)
        serr = float((np.abs(g_score[m] - o_score[m]) / np.maximum(1.0, np.abs(o_score[m]))).max()) if m.any() else 0.0
        # attention on the GPU's own selection at every sampled position
        g_o = o.float().cpu().numpy()[:, :, ts].astype(np.float64)
        r_o, _ = oracle.attention(op, data["q"], data["k"], data["v"], g_idx, ts=ts)
        aerr = float(np.abs(g_o - r_o).max())
        parity = {"positions": int(len(ts)), "non_exempt_mismatches": int((~same & ~exempt).sum()),
                  "exempt_fraction": round(float(exempt.mean()), 5), "exact_match_rate": round(float(same.mean()), 5),
                  "max_score_rel_err": serr, "max_attn_abs_err_on_gpu_selection": aerr,
                  "oracle_child_dots_per_query": cnt["child_dots"] / max(1, cnt["queries"]),
                  "oracle_leaf_pairs_per_query": cnt["leaf_pairs"] / max(1, cnt["queries"])}
        log(f"parity on sample: {parity}")

    return {
        "w": w, "steps": steps, "warmup": warmup, "ms_per_step": ms_per_step, "value": value,
        "select_ms": stage["pyramid"] + stage["select"], "flat_select_ms": flat_ms, "stage_ms": stage,
        "kernels": {kk: {"avg_ms": round(vv["avg_ms"], 4), "launches_per_step": vv["launches"] / steps}
                    for kk, vv in per_kernel.items()},
        "roofline": roofline, "kernel_rooflines": kernel_rooflines, "route_work": rc, "cpu_baseline": cpu,
        "parity": parity,
    }


def config_of(w) -> dict:
    return {"workload": w.name, "B": w.B, "N": w.N, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.D, "C": w.C, "g": 2,
            "K": w.K, "causal": w.causal, "needles": w.needles, "select": "two_stage"}


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards by KV head with no "
              "collective (each rank would run these kernels on its own KV heads)", file=sys.stderr)
        return 2
    import torch

    from hierarchical_block_sparse_mean_amd import inputs as I

    torch.cuda.set_device(0)
    if args.copy_calibration:  # first dispatch of the process: a plain 1 GiB device copy
        src = torch.zeros(1 << 29, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB read + 1 GiB write done")
        del src, dst
    if args.scaling:
        return scaling_main(args)
    if args.io:
        return io_main(args)
    if args.backward:
        return backward_main(args)
    w = I.workload(args.workload)
    if w.steps:
        return decode_main(args, w)
    ceilings = measured_ceilings()
    log(f"measured ceilings: {ceilings}")
    r = prefill_leg(args, w, ceilings, args.steps, args.warmup, cpu_leg=not args.no_cpu_baseline,
                    parity_positions=None)
    second = None
    if w.name == "prefill_128k" and not args.no_256k:
        # the metric's second sequence length, in the same process: fewer
        # steps (a 256K step is about five times a 128K one), no CPU leg, a
        # sampled parity summary
        torch.cuda.empty_cache()
        w2 = I.workload("prefill_256k")
        s2 = max(2, min(args.steps, 3))
        r2 = prefill_leg(args, w2, ceilings, s2, max(1, min(args.warmup, 1)), cpu_leg=False,
                         parity_positions=None if args.no_cpu_baseline else 96)
        second = {
            "config": config_of(w2), "steps": s2, "warmup": r2["warmup"], "value": round(r2["value"], 1),
            "unit": "tokens/s", "ms_per_step": round(r2["ms_per_step"], 4), "select_ms": round(r2["select_ms"], 4),
            "flat_select_ms": None if r2["flat_select_ms"] is None else round(r2["flat_select_ms"], 4),
            "stage_ms": {kk: round(vv, 4) for kk, vv in r2["stage_ms"].items()}, "kernels": r2["kernels"],
            "roofline": r2["roofline"], "kernel_rooflines": r2["kernel_rooflines"], "route_work": r2["route_work"],
            "parity": r2["parity"]}
    dec = None
    if w.name == "prefill_128k" and not args.no_decode:
        # the fused decode step on its own workload, in the same process: all
        # of its decode steps timed (a step is about a tenth of a millisecond),
        # its oracle parity sample kept small
        torch.cuda.empty_cache()
        wd = I.workload("decode_128k")
        d = decode_leg(wd, wd.steps, 8, cpu_leg=not args.no_cpu_baseline)
        dec = {kk: d[kk] for kk in ("metric", "config", "steps", "warmup", "value", "unit", "ms_per_step",
                                     "step_latency_ms", "kernels", "roofline", "cpu_baseline", "parity")}
    line = {
        "metric": METRIC,
        "value": round(r["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": config_of(w),
        "select_ms": round(r["select_ms"], 4),
        "flat_select_ms": None if r["flat_select_ms"] is None else round(r["flat_select_ms"], 4),
        "stage_ms": {kk: round(vv, 4) for kk, vv in r["stage_ms"].items()},
        "timing_note": "value, ms_per_step and stage_ms: the K timed steps (stage events only); kernels and "
                       "rooflines: the same K steps re-run with HIP events around every launch",
        "kernels": r["kernels"],
        "roofline": r["roofline"],
        "kernel_rooflines": r["kernel_rooflines"],
        "measured_ceilings": ceilings,
        "route_work": r["route_work"],
        "cpu_baseline": r["cpu_baseline"],
        "parity": r["parity"],
        "prefill_256k": second,
        "decode_128k": dec,
    }
    print(json.dumps(line), flush=True)
    return 0


def scaling_parity(w, data, idx, score, o, n_pos: int) -> dict:
    """The GPU's selection (idx, score: tensors or host arrays of the whole
    problem) and, unless o is None, its attention, at n_pos sampled
    positions (the first and last leaves included) against the oracle:
    non-exempt set mismatches (sets must match except where the oracle's
    K-th and (K+1)-th scores at some scored level are within 1e-3),
    reported-score error, and attention on the GPU's own selection."""
    import numpy as np

    import oracle

    host = lambda x: x if isinstance(x, np.ndarray) else x.cpu().numpy()
    rng = np.random.default_rng(w.N)
    ts = np.unique(np.concatenate([[0, w.C - 1, w.C, w.N - 1], rng.integers(0, w.N, n_pos)]))
    op = oracle.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=w.causal)
    r_idx, r_score, r_gap, _ = oracle.select(op, data["q"], data["k"], ts=ts)
    g_idx = host(idx)[:, :, ts]
    g_score = host(score)[:, :, ts].astype(np.float64)
    same = (g_idx == r_idx).all(-1)
    exempt = r_gap < 1e-3
    m = same[..., None] & (r_idx >= 0)
    serr = float((np.abs(g_score[m] - r_score[m]) / np.maximum(1.0, np.abs(r_score[m]))).max()) if m.any() else 0.0
    out = {"positions": int(len(ts)), "non_exempt_mismatches": int((~same & ~exempt).sum()),
           "exempt_fraction": round(float(exempt.mean()), 4), "exact_match_rate": round(float(same.mean()), 4),
           "max_score_rel_err": serr}
    if o is not None:
        r_o, _ = oracle.attention(op, data["q"], data["k"], data["v"], g_idx, ts=ts)
        out["max_attn_abs_err_on_gpu_selection"] = float(
            np.abs(o.float().cpu().numpy()[:, :, ts].astype(np.float64) - r_o).max())
    return out


def scaling_main(args) -> int:
    """Selection time against N at fixed C = 64, K = 16 (Hq = 32, Hkv = 8,
    d = 128, bf16, causal, planted needle leaves as in the 32K/128K workloads):
    pyramid + two-stage select, the flat selector, and attention, each timed
    with HIP events over --steps repetitions after one warm-up, then each N's
    selection and attention checked against the oracle on sampled positions.
    Prints one JSON line with the table, log-log slopes and the interpolated
    N where the flat selector becomes slower than PISA's."""
    import numpy as np
    import torch

    from hierarchical_block_sparse_mean_amd import inputs as I
    from hierarchical_block_sparse_mean_amd import pisa

    rows = []
    for N in [int(x) for x in args.scaling_n.split(",")]:
        w = I.Workload(f"scaling_{N // 1024}k", 1, N, 32, 8, 128, 64, 16, "bf16", True, "leaf_per_query", seed=5000)
        t0 = time.perf_counter()
        data = I.generate(w)
        q, k, v = dev(data["q"]), dev(data["k"]), dev(data["v"])
        log(f"N={N}: inputs ready in {time.perf_counter() - t0:.1f}s")
        p = pisa.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=True, dtype="bf16")
        pyr = pisa.alloc_pyramid(p)
        ws = pisa.workspace(pisa.select_workspace_bytes(p))
        aws = pisa.workspace(pisa.attn_workspace_bytes(p))
        idx = torch.empty((w.B, w.Hkv, w.N, w.K), dtype=torch.int32, device="cuda")
        score = torch.empty_like(idx, dtype=torch.float32)
        fidx = torch.empty_like(idx)
        fscore = torch.empty_like(score)
        fws = pisa.workspace(pisa.flat_workspace_bytes(p))
        o = torch.empty_like(q)

        def timed(fn):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.steps

        def sel():
            pisa.build_pyramid(p, k, pyr)
            pisa.select(p, q, k, pyr, idx=idx, score=score, ws=ws)

        def flat():
            pisa.build_pyramid(p, k, pyr)
            pisa.flat_select(p, q, pyr, idx=fidx, score=fscore, ws=fws)

        sel_ms = timed(sel)
        flat_ms = timed(flat)
        attn_ms = timed(lambda: pisa.sparse_attn(p, q, k, v, idx, o=o, lse=None, ws=aws, with_lse=False))
        rc = pisa.route_counts(p, q, k, pyr)
        # sampled check of this N's selection and attention against the oracle
        # (the timed calls above left their outputs in idx, score and o)
        sel()
        pisa.sparse_attn(p, q, k, v, idx, o=o, lse=None, ws=aws, with_lse=False)
        torch.cuda.synchronize()
        par = scaling_parity(w, data, idx, score, o, args.scaling_positions)
        rows.append({"N": N, "levels": pisa.levels(N, w.C), "select_ms": round(sel_ms, 4),
                     "flat_select_ms": round(flat_ms, 4), "attention_ms": round(attn_ms, 4),
                     "step_ms": round(sel_ms + attn_ms, 4),
                     "child_rows_per_query": round(rc["child_rows"] / max(1, rc["queries"]), 2),
                     "flat_leaves_per_query": round((pisa.level_rows(N, w.C, 1) + 1) / 2, 1),
                     "parity": par})
        log(f"N={N}: select {sel_ms:.3f} ms, flat {flat_ms:.3f} ms, attention {attn_ms:.3f} ms; parity {par}")
        del q, k, v, pyr, ws, aws, idx, score, fidx, fscore, fws, o, data
        torch.cuda.empty_cache()
    ln = np.log([r["N"] for r in rows])
    slope = lambda key: float(np.polyfit(ln, np.log([r[key] for r in rows]), 1)[0]) if len(rows) > 1 else None
    # first N where flat is slower, interpolated in log N between neighbours
    cross = None
    ratio = [r["flat_select_ms"] / r["select_ms"] for r in rows]
    for i in range(1, len(rows)):
        if ratio[i - 1] < 1.0 <= ratio[i]:
            a, b = math.log(ratio[i - 1]), math.log(ratio[i])
            f = -a / (b - a)
            cross = round(math.exp(ln[i - 1] + f * (ln[i] - ln[i - 1])))
    line = {
        "metric": "PISA select vs flat select scaling (C=64, K=16), 1 GPU",
        "value": cross,
        "unit": "tokens (crossover N; null if not reached)",
        "n_gpus": 1,
        "steps": args.steps,
        "higher_is_better": False,
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "scaling", "B": 1, "Hq": 32, "Hkv": 8, "d": 128, "C": 64, "g": 2, "K": 16,
                   "causal": True, "needles": "leaf_per_query"},
        "rows": rows,
        "loglog_slope": {"select_ms": slope("select_ms"), "flat_select_ms": slope("flat_select_ms"),
                         "attention_ms": slope("attention_ms")},
        "flat_over_select": [round(x, 4) for x in ratio],
    }
    print(json.dumps(line), flush=True)
    return 0


def backward_main(args) -> int:
    """Sparse-attention backward over the selection of the workload's
    queries: forward (with lse) then backward with a seeded N(0,1) output
    gradient, each timed with HIP events over --steps repetitions.  Work:
    attention forward 4 d flop per attended (query head, key); backward
    10 d (S recomputed, dP, dV, dK, dQ)."""
    import numpy as np
    import torch

    from hierarchical_block_sparse_mean_amd import inputs as I
    from hierarchical_block_sparse_mean_amd import pisa

    w = I.workload(args.workload)
    data = I.generate(w)
    q, k, v = dev(data["q"]), dev(data["k"]), dev(data["v"])
    g = dev(I.normal(w.seed, 11, w.B * w.Hq * w.N * w.D, dtype=w.dtype).reshape(w.B, w.Hq, w.N, w.D))
    del data
    p = pisa.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=w.causal, dtype=w.dtype)
    pyr = pisa.build_pyramid(p, k)
    idx, _ = pisa.select(p, q, k, pyr)
    aws = pisa.workspace(pisa.attn_workspace_bytes(p))
    bws = pisa.workspace(pisa.attn_backward_workspace_bytes(p))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.zeros_like(k), torch.zeros_like(v)

    def fwd():
        pisa.sparse_attn(p, q, k, v, idx, o=o, lse=lse, ws=aws)

    def bwd():
        pisa.sparse_attn_backward(p, q, k, v, idx, o, lse, g, dq=dq, dk=dk, dv=dv, ws=bws)

    fwd()
    bwd()
    torch.cuda.synchronize()
    res = {}
    kern = {}
    for name, fn in (("forward", fwd), ("backward", bwd)):
        pisa.timer_enable(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        kern[name] = {kk: {"avg_ms": round(vv[1] / max(1, vv[0]), 4), "launches_per_step": vv[0] / args.steps}
                      for kk, vv in pisa.timer_report().items()}
        pisa.timer_enable(False)
        res[name] = e0.elapsed_time(e1) / args.steps
        log(f"{name}: {res[name]:.3f} ms")
    keys = attended_keys(idx, w.N, w.C, w.causal) * (w.Hq // w.Hkv)
    fwd_tf = 4.0 * w.D * keys / (res["forward"] * 1e-3) / 1e12
    bwd_tf = 10.0 * w.D * keys / (res["backward"] * 1e-3) / 1e12
    line = {
        "metric": "PISA sparse-attention backward ms over the prefill selection, 1 GPU",
        "value": round(res["backward"], 4), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "higher_is_better": False, "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.D, "C": w.C, "g": 2,
                   "K": w.K, "causal": w.causal},
        "forward_ms": round(res["forward"], 4),
        "attended_head_keys": int(keys),
        "roofline": {"forward": {"bound": "mfma", "achieved_TFLOPs": round(fwd_tf, 2),
                                 "frac": round(fwd_tf / PEAK["mfma_bf16_TFLOPs"], 5)},
                     "backward": {"bound": "mfma", "achieved_TFLOPs": round(bwd_tf, 2),
                                  "frac": round(bwd_tf / PEAK["mfma_bf16_TFLOPs"], 5)}},
        "kernels": kern,
    }
    print(json.dumps(line), flush=True)
    return 0


def io_main(args) -> int:
    """One-stage (fused descent to raw-key leaves, one program per query and
    KV head) against two-stage selection (stage-1 routing, clusters, MFMA leaf
    scoring over shared key tiles, final top-K) at G_Q = 4 (Hkv = 8) and
    G_Q = 16 (Hkv = 2), Hq = 32, N = 131072, C = 64, K = 16, bf16, causal,
    planted needle leaves.  Times each schedule with HIP events (pyramid
    included), compares their selections, and gives the leaf-level bytes per
    (query, candidate leaf) of the pages' IO comparison (one-stage: C key rows;
    two-stage: G_Q query rows + C / Q_tile key rows, Q_tile = 4) next to this
    design's (G_Q query rows + 2C key rows shared by the queries of a cluster
    chunk).  Both schedules' selections are checked against the oracle at
    sampled positions (--scaling-positions of them) for each G_Q."""
    import numpy as np
    import torch

    from hierarchical_block_sparse_mean_amd import inputs as I
    from hierarchical_block_sparse_mean_amd import pisa

    rows = []
    for hkv in (8, 2):
        G = 32 // hkv
        w = I.Workload(f"io_g{G}", 1, 131072, 32, hkv, 128, 64, 16, "bf16", True, "leaf_per_query", seed=2000)
        data = I.generate(w, with_v=False)
        q, k = dev(data["q"]), dev(data["k"])
        out = {}
        # two-stage at both Q_tile values (queries sharing one read of a key
        # fragment from LDS: one 16-column MFMA tile = 16/G_Q, two = 32/G_Q)
        for algo, name, qt in ((pisa.SELECT_TWO_STAGE, "two_stage", 32 // G),
                               (pisa.SELECT_TWO_STAGE, "two_stage_q16", 16 // G),
                               (pisa.SELECT_FUSED, "one_stage", 0)):
            p = pisa.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=True, dtype="bf16", select_algo=algo,
                             q_tile=qt)
            pyr = pisa.alloc_pyramid(p)
            ws = pisa.workspace(pisa.select_workspace_bytes(p))
            idx = torch.empty((w.B, w.Hkv, w.N, w.K), dtype=torch.int32, device="cuda")
            score = torch.empty_like(idx, dtype=torch.float32)

            def run():
                pisa.build_pyramid(p, k, pyr)
                pisa.select(p, q, k, pyr, idx=idx, score=score, ws=ws)

            run()
            torch.cuda.synchronize()
            pisa.timer_enable(True)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                run()
            e1.record()
            torch.cuda.synchronize()
            kern = pisa.timer_report()
            pisa.timer_enable(False)
            out[name] = {"ms": e0.elapsed_time(e1) / args.steps, "idx": idx.cpu().numpy(),
                         "score": score.cpu().numpy(),
                         "kernels": {kk: round(vv[1] / max(1, vv[0]), 4) for kk, vv in kern.items()}}
            log(f"G_Q={G} {name}: {out[name]['ms']:.3f} ms {out[name]['kernels']}")
            del pyr, ws, idx, score
        # (query, candidate leaf) pairs both schedules score: the two leaves of
        # every level-2 block stage 1 keeps
        pc = pisa.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=True, dtype="bf16")
        pyr_c = pisa.build_pyramid(pc, k)
        rc = pisa.route_counts(pc, q, k, pyr_c)
        del pyr_c
        same = float((out["two_stage"]["idx"] == out["one_stage"]["idx"]).all(-1).mean())
        same_qt = bool(np.array_equal(out["two_stage"]["idx"], out["two_stage_q16"]["idx"]))
        parity = {nm: scaling_parity(w, data, out[nm]["idx"], out[nm]["score"], None, args.scaling_positions)
                  for nm in ("two_stage", "one_stage")}
        log(f"G_Q={G} oracle check: {parity}")
        d, C, qt, chunk = w.D, w.C, 4, 1024
        rows.append({
            "G_Q": G, "Hkv": hkv,
            "two_stage_ms": round(out["two_stage"]["ms"], 4), "one_stage_ms": round(out["one_stage"]["ms"], 4),
            "two_stage_kernels_ms": out["two_stage"]["kernels"], "one_stage_kernels_ms": out["one_stage"]["kernels"],
            "same_selection_rate": round(same, 5),
            "parity": parity,
            "queries": rc["queries"], "candidate_leaf_pairs": 2 * rc["kept_level2"],
            "q_tile_sweep": {
                "q_tile": [16 // G, 32 // G],
                "leaf_score_ms": [out["two_stage_q16"]["kernels"].get("leaf_score"),
                                  out["two_stage"]["kernels"].get("leaf_score")],
                "lds_key_bytes_per_pair": [2 * C * d * 2 * G // 16, 2 * C * d * 2 * G // 32],
                "identical_selection": same_qt},
            "leaf_bytes_per_pair": {"one_stage": C * d * 2, "two_stage_pages": (G + C // qt) * d * 2,
                                    "two_stage_here": round(G * d * 2 + 2 * C * d * 2 / chunk, 1)},
        })
        del q, k, data
        torch.cuda.empty_cache()
    line = {
        "metric": "PISA one-stage vs two-stage selection ms at N=131072, G_Q in {4, 16}, 1 GPU",
        "value": rows[-1]["two_stage_ms"], "unit": "ms (two-stage, G_Q = 16)", "n_gpus": 1, "steps": args.steps,
        "higher_is_better": False, "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "io", "B": 1, "N": 131072, "Hq": 32, "d": 128, "C": 64, "g": 2, "K": 16,
                   "causal": True, "needles": "leaf_per_query"},
        "rows": rows,
    }
    print(json.dumps(line), flush=True)
    return 0


def decode_bytes_model(n: int, C: int, K: int, D: int, G: int, esz: int) -> dict:
    """Algorithmic HBM bytes of one fused decode step for one (sequence, KV
    head) whose prefix holds n tokens after the append.  Candidate counts
    follow the descent with every block valid (the new query sees the whole
    prefix): one root candidate, at each level the children of the kept
    blocks; a level with more than K candidates is scored.  Children counts
    assume full sibling pairs, so they may exceed the kernel's by one row per
    level at a ragged tail."""
    rows = [-(-n // C)]
    while rows[-1] > 1:
        rows.append(-(-rows[-1] // 2))
    L = len(rows)  # rows[l-1] = M_l
    summary_rows = 0
    a = 1
    for l in range(L, 1, -1):
        if a > K:
            summary_rows += min(2 * a, rows[l - 2])
        kept = min(a, K)
        a = min(2 * kept, rows[l - 2])
    leaf_keys = (a if a > K else 0) * C          # level-1 candidates scored on raw keys
    kept_keys = min(a, K) * C
    lo = (n - 1) // C * C
    b = {
        "q_o": 2 * G * D * esz,
        "append": 2 * D * esz,
        "leaf_mean": (n - 1 - lo) * D * esz,
        "path": (L - 1) * D * 4 + L * (D * 4 + D * 2 + 4),
        "summaries": summary_rows * (D * 2 + 4),  # fp16 block-floating-point rows and their exponents
        "leaf_keys": max(leaf_keys, kept_keys) * D * esz,  # keys of the scored (or kept) leaves, read once
        "values": kept_keys * D * esz,
        "idx": 2 * K * 4,
    }
    b["total"] = sum(b.values())
    b["levels"] = L
    b["summary_rows"] = summary_rows
    return b


def decode_leg(w, steps: int, warmup: int, cpu_leg: bool) -> dict:
    """Fused decode: S sequences with an N-token cached prefix; one step
    appends one token per sequence (k, v, leaf mean, ancestor path) and runs
    selection + sparse attention for it in one kernel.  The timed region is
    K consecutive steps starting from the N-token prefix."""
    import numpy as np
    import torch

    from hierarchical_block_sparse_mean_amd import inputs as I
    from hierarchical_block_sparse_mean_amd import pisa

    if steps > w.steps or warmup > w.steps:
        raise SystemExit(f"{w.name} has {w.steps} decode steps; asked for --steps {steps} --warmup {warmup}")
    S, cap, G = w.B, w.N + w.steps, w.Hq // w.Hkv
    log(f"workload {w.name}: S={S} sequences x N={w.N} cached tokens (+{w.steps} steps), Hq={w.Hq} Hkv={w.Hkv} "
        f"D={w.D} C={w.C} K={w.K} {w.dtype}")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    kc = torch.zeros((S, w.Hkv, cap, w.D), dtype=dt, device="cuda")
    vc = torch.zeros_like(kc)
    t0 = time.perf_counter()
    for s in range(S):
        kh, vh = I.decode_prefix(w, s)
        kc[s, :, : w.N].copy_(dev(kh))
        vc[s, :, : w.N].copy_(dev(vh))
        if s % 16 == 15:
            log(f"cache: {s + 1}/{S} sequences generated and uploaded ({time.perf_counter() - t0:.1f}s)")
    del kh, vh
    toks = [I.decode_token(w, st) for st in range(w.steps)]
    tq = dev(np.stack([t["q"] for t in toks]))
    tk = dev(np.stack([t["k"] for t in toks]))
    tv = dev(np.stack([t["v"] for t in toks]))
    log(f"inputs ready in {time.perf_counter() - t0:.1f}s")

    dp = pisa.DecodeProblem(S, cap, w.Hq, w.Hkv, w.D, w.C, w.K, dtype=w.dtype)
    pp = dp.prefill_problem(w.N)
    pyr = pisa.alloc_pyramid(pp)
    length = torch.empty((S,), dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o_all = torch.empty((w.steps, S, w.Hq, w.D), dtype=dt, device="cuda")
    idx_all = torch.empty((w.steps, S, w.Hkv, w.K), dtype=torch.int32, device="cuda")
    score_all = torch.empty((w.steps, S, w.Hkv, w.K), dtype=torch.float32, device="cuda")

    def reset():
        length.fill_(w.N)
        pisa.build_pyramid(pp, kc, pyr)

    def step(i):
        pisa.decode_step(dp, kc, vc, pyr, length, tq[i], tk[i], tv[i], o=o_all[i], idx=idx_all[i],
                         score=score_all[i], err=err)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    reset()
    e1.record()
    torch.cuda.synchronize()
    pyr_ms = e0.elapsed_time(e1)
    log(f"prefix pyramid built in {pyr_ms:.3f} ms")
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    log(f"warmup {warmup} steps done; cache length and pyramid reset to the prefix")

    # timed region: the K steps alone.  At this step length, HIP events around
    # every launch and step would cost about a sixth of the step, so the
    # kernel times and step latencies come from a second pass: the same K
    # steps again from the reset prefix, with the library timer and per-step
    # events on the launch stream.
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    if int(err.item()) != 0:
        raise SystemExit("decode reported a full cache")
    ms_per_step = wall * 1000.0 / steps
    value = S * steps / wall
    reset()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    pisa.timer_enable(True)
    for i in range(steps):
        evs[i][0].record()
        step(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    kernels = pisa.timer_report()
    pisa.timer_enable(False)
    if int(err.item()) != 0:
        raise SystemExit("decode reported a full cache")
    lat = np.array([a.elapsed_time(b) for a, b in evs])
    log(f"timed {steps} steps: {ms_per_step:.4f} ms/step; instrumented pass: median step {np.median(lat):.4f} ms, "
        f"p99 {np.percentile(lat, 99):.4f} ms")
    per_kernel = {kk: {"launches": vv[0], "avg_ms": vv[1] / max(1, vv[0])} for kk, vv in kernels.items()}

    # roofline of the fused decode kernel, on the modelled bytes of each step
    esz = 2 if w.dtype == "bf16" else 4
    per_launch = 0
    for i in range(steps):
        per_launch += decode_bytes_model(w.N + i + 1, w.C, w.K, w.D, G, esz)["total"] * S * w.Hkv
    per_launch /= steps
    mid = decode_bytes_model(w.N + 1, w.C, w.K, w.D, G, esz)
    dk = per_kernel.get("decode")
    roofline = None
    if dk:
        ach = per_launch / (dk["avg_ms"] * 1e-3) / 1e9
        roofline = {"kernel": "decode", "bound": "hbm", "achieved": round(ach, 2), "peak": PEAK["hbm_GBps"],
                    "unit": "GB/s", "frac": round(ach / PEAK["hbm_GBps"], 5), "traffic": traffic_for("decode", w.name),
                    "avg_launch_ms": round(dk["avg_ms"], 5), "work_per_launch": round(per_launch, 1),
                    "work_note": f"modelled bytes per (sequence, KV head) at n={w.N + 1}: {mid}"}
        if roofline["traffic"]:
            roofline["traffic_GBps"] = round(roofline["traffic"] / (dk["avg_ms"] * 1e-3) / 1e9, 1)

    # CPU oracle on a few sequences at the first and last timed step, with parity
    cpu = parity = None
    if cpu_leg:
        import oracle

        seqs = [0, S // 3, (2 * S) // 3, S - 1][: max(1, min(4, S))]
        checks = sorted({0, steps - 1})
        g_idx = idx_all.cpu().numpy()
        g_score = score_all.cpu().numpy().astype(np.float64)
        g_o = o_all.float().cpu().numpy().astype(np.float64)
        t_cpu, n_tok = 0.0, 0
        nonex = mism = total = 0
        exempt_n = 0
        serr = aerr = 0.0
        for s in seqs:
            kh, vh = I.decode_prefix(w, s)
            for st in checks:
                n = w.N + st + 1
                kp = np.empty((1, w.Hkv, n, w.D), kh.dtype)
                vp = np.empty_like(kp)
                kp[0, :, : w.N], vp[0, :, : w.N] = kh, vh
                for j in range(st + 1):
                    kp[0, :, w.N + j], vp[0, :, w.N + j] = toks[j]["k"][s], toks[j]["v"][s]
                ta = time.perf_counter()
                r_idx, r_score, r_gap, r_o, _ = oracle.decode_reference(
                    oracle.Problem(1, n, w.Hq, w.Hkv, w.D, w.C, w.K, causal=True), toks[st]["q"][s:s + 1], kp, vp)
                t_cpu += time.perf_counter() - ta
                n_tok += 1
                same = (g_idx[st, s] == r_idx[0]).all(-1)
                exempt = r_gap[0] < 1e-3
                total += same.size
                mism += int((~same).sum())
                nonex += int((~same & ~exempt).sum())
                exempt_n += int(exempt.sum())
                m = same[:, None] & (r_idx[0] >= 0)
                if m.any():
                    serr = max(serr, float((np.abs(g_score[st, s][m] - r_score[0][m]) /
                                            np.maximum(1.0, np.abs(r_score[0][m]))).max()))
                okh = np.repeat(same, G)
                if okh.any():
                    aerr = max(aerr, float(np.abs(g_o[st, s] - r_o[0]).max(-1)[okh].max()))
        cpu = {"value": round(n_tok / t_cpu, 3), "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
               "sample": f"{n_tok} decode tokens: sequences {seqs} at steps {checks}; the oracle rebuilds the "
                         f"prefix pyramid per (sequence, KV head) then selects and attends, fp64, {t_cpu:.1f}s wall"}
        parity = {"tokens": n_tok, "heads": total, "non_exempt_mismatches": nonex, "exempt": exempt_n,
                  "exact_match_rate": round(1.0 - mism / max(1, total), 5), "max_score_rel_err": serr,
                  "max_attn_abs_err": aerr}
        log(f"parity on sample: {parity}")

    line = {
        "metric": "PISA fused decode tokens/s (selection + sparse attention per new token), 1 GPU",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "S": S, "N": w.N, "decode_steps": w.steps, "Hq": w.Hq, "Hkv": w.Hkv,
                   "d": w.D, "C": w.C, "g": 2, "K": w.K},
        "step_latency_ms": {"median": round(float(np.median(lat)), 5), "p99": round(float(np.percentile(lat, 99)), 5),
                            "min": round(float(lat.min()), 5), "max": round(float(lat.max()), 5)},
        "prefix_pyramid_ms": round(pyr_ms, 4),
        "timing_note": "value and ms_per_step: the K steps with nothing else on the stream; kernels, roofline and "
                       "step_latency_ms: the same K steps re-run from the prefix with HIP events per launch and step",
        "kernels": {kk: {"avg_ms": round(vv["avg_ms"], 5), "launches_per_step": vv["launches"] / steps}
                    for kk, vv in per_kernel.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    return line


def decode_main(args, w) -> int:
    print(json.dumps(decode_leg(w, args.steps, args.warmup, not args.no_cpu_baseline)), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
