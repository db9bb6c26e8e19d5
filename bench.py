#!/usr/bin/env python3
"""Benchmark of the MSA main-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input that
is already resident in HBM: schedule build (selection cleaning, k2q CSR,
task table), sparse forward, backward preprocess, backward main kernel
(KV-parallel: S^T, dP^T, dV, dK, and in the default dq mode "ds" each tile's
dS stored), backward dQ kernel (query-parallel: dQ from the stored dS, or
recomputing S^T and dP^T in mode "recompute"), backward postprocess.
Workload: one 8192-token document, 4 KV heads x 16 query heads, head dim
128, key block 64, 8-query chunks, top-k 16.

Prints one JSON line.  ``value`` is useful TFLOP/s of forward + backward:
every selected (index head, chunk, block) pair counts as one 128 x 64 tile,
2 contractions forward and 5 backward, each 2*128*64*128 FLOPs; recomputed
contractions are not counted.  The warmup steps carry a HIP event between
every two kernels, which picks the kernel with the largest time; the timed
K steps that follow carry events only around that kernel, whose mean launch
duration (HIP events on torch's current stream, the stream the kernels are
launched on) gives the ``roofline`` object; K more steps with events
between all kernels then give the per-kernel breakdown.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6          # MI355X dense bf16 MFMA: 256 CUs x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
WORKLOAD = "single8k"
KERNEL_FILES = {"forward": "forward.hip", "bwd_main": "backward.hip", "bwd_dq": "dq.hip"}
KERNEL_FILES_RECOMPUTE = dict(KERNEL_FILES, bwd_dq="dq_recompute.hip")
KERNEL_NAMES = {  # per dq mode
    "recompute": {"forward": "forward_kernel<128>", "bwd_main": "backward_kv_kernel<128, false, 1>",
                  "bwd_dq": "dq_kernel<128>"},
    "ds": {"forward": "forward_kernel<128>", "bwd_main": "backward_kv_kernel<128, true, 1>",
           "bwd_dq": "dq_from_ds_kernel<128>"},
    "atomic": {"forward": "forward_kernel<128>", "bwd_main": "backward_main_kernel<128, false>"},
    "atomic_bf16": {"forward": "forward_kernel<128>", "bwd_main": "backward_main_kernel<128, true>"},
    # key block 128: the KV-parallel kernel holds both 64-key tiles of a block
    # in one 8-wave workgroup; the pool kernel takes them on two workgroups
    "ds_b128": {"forward": "forward_kernel<128>", "bwd_main": "backward_kv_kernel<128, true, 2>",
                "bwd_dq": "dq_from_ds_kernel<128>"},
    "recompute_b128": {"forward": "forward_kernel<128>", "bwd_main": "backward_kv_kernel<128, false, 2>",
                       "bwd_dq": "dq_kernel<128>"},
    "atomic_b128": {"forward": "forward_kernel<128>", "bwd_main": "backward_main_kernel<128, false>"},
    "atomic_bf16_b128": {"forward": "forward_kernel<128>", "bwd_main": "backward_main_kernel<128, true>"},
}


def pair_flops(block: int, head_dim: int) -> tuple[int, int]:
    tile = 2 * 128 * block * head_dim
    return 2 * tile, 5 * tile


def kernel_source_hash(kernel: str, mode: str = "ds") -> str:
    """Hash of what the kernel is built from: its source file, the shared
    device header and the compiler flags that file gets."""
    from block_sparse_attention_k2q_amd import build as msa_build
    h = hashlib.sha256()
    files = KERNEL_FILES_RECOMPUTE if mode.startswith("recompute") else KERNEL_FILES
    for rel in (files[kernel], "msa_device.h"):
        with open(os.path.join(ROOT, "block_sparse_attention_k2q_amd", "csrc", rel), "rb") as f:
            h.update(f.read())
    flags = msa_build.FLAGS + msa_build.PER_SOURCE_FLAGS.get(files[kernel], [])
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def traffic_profile_path(kernel_name: str) -> str:
    """profiles/<kernel>_<workload>_hbm_traffic.md for a kernel name such as
    'dq_kernel<128>' (non-alphanumerics become underscores)."""
    stem = re.sub(r"[^A-Za-z0-9]+", "_", kernel_name).strip("_")
    return os.path.join(ROOT, "profiles", f"{stem}_{WORKLOAD}_hbm_traffic.md")


def measured_traffic(kernel: str, mode: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 --pmc
    summary, or None when absent or taken on a different kernel source."""
    try:
        with open(traffic_profile_path(KERNEL_NAMES[mode][kernel])) as f:
            text = f.read()
    except OSError:
        return None
    src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not src or not val or src.group(1) != kernel_source_hash(kernel, mode):
        return None
    return float(val.group(1))


def _oracle_share(job):
    """One worker's share of the CPU baseline, in a fresh process with one
    BLAS thread: the fp64 oracle (forward + backward) on the given
    (index head, chunk) pairs; returns its own wall time."""
    paths, cu, sel_clean, block, scale, chunks = job
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import msa_oracle as O
    q, k, v, do = (np.load(path, mmap_mode="r") for path in paths)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        O.backward_gathered(q, k, v, do, cu, sel_clean, block, scale, chunks=chunks)
        return time.perf_counter() - t0


def _noop(x):
    return x


def cpu_baseline(w, sched_host, max_pairs: int = 8192) -> dict:
    """The fp64 oracle on the host cores: the workload's (index head, chunk)
    pairs (all of them, or an even spread of max_pairs), forward + backward
    of each, sharded over one worker process per core (one BLAS thread
    each), reported in useful TFLOP/s over the wall time of the sharded run.
    The workers read fp32 copies of q, k, v, dO (the bf16 values, exact)
    from memory-mapped files; every oracle call widens them to fp64 itself."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import shutil
    import tempfile
    import numpy as np
    cores = len(os.sched_getaffinity(0))
    lay = sched_host["layout"]
    sel_clean = sched_host["sel_clean"]
    pairs_all = [(i, g) for g in range(lay.C) for i in range(w.num_kv_heads) if (sel_clean[i, g] >= 0).any()]
    if len(pairs_all) > max_pairs:
        pick = np.linspace(0, len(pairs_all) - 1, max_pairs).astype(int)
        pairs_all = [pairs_all[x] for x in pick]
    # each worker holds fp64 q, dO and the dq, out it writes: 32 bytes per element of q
    per_worker = 32 * w.q.numel()
    workers = max(1, min(cores, len(pairs_all), int((96 << 30) // per_worker)))
    shares = [pairs_all[x::workers] for x in range(workers)]
    tmp = tempfile.mkdtemp(prefix="msa_baseline_")
    try:
        paths = []
        for name, t in (("q", w.q), ("k", w.k), ("v", w.v), ("do", w.do)):
            path = os.path.join(tmp, name + ".npy")
            np.save(path, t.float().numpy())
            paths.append(path)
        jobs = [(paths, w.cu_seqlens, sel_clean, w.block, w.scale, share) for share in shares]
        # fresh interpreters (no GPU state inherited); a worker that dies
        # fails the run instead of being restarted
        with cf.ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn")) as pool:
            list(pool.map(_noop, range(workers)))      # workers started and imported
            t0 = time.perf_counter()
            list(pool.map(_oracle_share, jobs))
            dt = time.perf_counter() - t0
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    blocks = int(sum((sel_clean[i, g] >= 0).sum() for i, g in pairs_all))
    fwd_f, bwd_f = pair_flops(w.block, w.head_dim)
    n_all = int(sum((sel_clean[i, g] >= 0).any() for g in range(lay.C) for i in range(w.num_kv_heads)))
    what = "all" if len(pairs_all) == n_all else f"an even spread of {len(pairs_all)} of the {n_all}"
    return {"value": blocks * (fwd_f + bwd_f) / dt / 1e12, "unit": "TFLOP/s", "cores": workers,
            "kind": "oracle",
            "sample": f"{what} (index head, chunk) pairs of the {WORKLOAD} workload ({blocks} selected "
                      f"blocks), fp64 forward+backward, sharded over {workers} worker processes with one "
                      f"BLAS thread each, {dt:.1f} s wall"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dq-mode", choices=("ds", "recompute", "atomic", "atomic_bf16"), default="ds")
    ap.add_argument("--block", type=int, choices=(64, 128), default=64,
                    help="key block size: 64 (the headline workload) or 128 (the same workload at the "
                         "pages' production block size)")
    ap.add_argument("--workload", choices=("single8k", "varlen8", "long64k", "zipf16k"), default="single8k",
                    help="single8k is the headline workload; the others are the remaining full-size "
                         "configurations (packed varlen, 64k context at top-32, Zipf-skewed selection)")
    ap.add_argument("--forward", choices=("query", "kv"), default="query",
                    help="query: the query-parallel forward (default); kv: the planner-driven forward that "
                         "walks the task table (KV-parallel, exact cross-workgroup softmax merge)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed steps, run a plain device-to-device copy of this many MiB "
                         "three times (the known-size reference for HBM byte counters)")
    args = ap.parse_args()
    global WORKLOAD
    WORKLOAD = args.workload
    if args.block == 128:
        WORKLOAD = args.workload + "_b128"
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this library has no multi-GPU "
              "path: the method shards by KV head with no exchange, see the design notes.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from block_sparse_attention_k2q_amd import binding as B
    from block_sparse_attention_k2q_amd.workloads import make_workload

    dev = torch.device("cuda", 0)
    num_cus = B.msa_device_check(0)
    w = make_workload(args.workload, block=args.block)
    dq_mode = {"recompute": B.DQ_RECOMPUTE, "ds": B.DQ_DS_BUFFER, "atomic": B.DQ_ATOMIC_POOL,
               "atomic_bf16": B.DQ_ATOMIC_POOL_BF16}[args.dq_mode]
    p = B.Problem.make(w.cu_seqlens, w.num_kv_heads, w.head_dim, w.topk, num_cus=num_cus,
                       softmax_scale=w.scale, block_size=w.block, dq_mode=dq_mode)
    q, k, v, do = (x.to(dev) for x in (w.q, w.k, w.v, w.do))
    cu = torch.from_numpy(w.cu_seqlens).to(dev)
    sel = torch.from_numpy(w.sel).to(dev)
    sched = B.alloc_schedule(p, dev)
    scratch = B.alloc_scratch(p, dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if args.forward == "kv":
        fwd_scratch = torch.empty(B.msa_forward_kv_scratch_bytes(p), dtype=torch.uint8, device=dev)

        def run_forward():
            B.msa_forward_kv(p, q, k, v, cu, sched, fwd_scratch, out, lse)
    else:
        def run_forward():
            B.msa_forward(p, q, k, v, cu, sched, out, lse)

    names = ("schedule", "forward", "bwd_pre", "bwd_main", "bwd_dq", "bwd_post")

    def step(ev=None, marks=range(7)):
        def mark(x):
            if ev is not None and x in marks:
                ev[x].record()
        mark(0)
        B.msa_build_schedule(p, cu, sel, sched)
        mark(1)
        run_forward()
        mark(2)
        B.msa_backward_preprocess(p, out, do, scratch)
        mark(3)
        B.msa_backward_main(p, q, k, v, do, lse, cu, sched, scratch)
        mark(4)
        B.msa_backward_dq(p, q, k, v, do, lse, cu, sched, scratch, dq)
        mark(5)
        B.msa_backward_postprocess(p, sched, scratch, dq, dk, dv)
        mark(6)

    def event_rows(n):
        return [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(n)]

    # Warmup, with an event between every two kernels: the kernel with the
    # largest time gets the events of the timed steps.
    wev = event_rows(args.warmup)
    for s in range(args.warmup):
        step(wev[s])
    torch.cuda.synchronize()
    # The choice uses the last warmup step: the first launch of each kernel
    # also loads its code, so with a single warmup step the main backward
    # kernel (4 of the 7 contractions per pair) is taken.
    timed = {"forward": 1, "bwd_main": 3, "bwd_dq": 4}
    dominant = "bwd_main" if len(wev) < 2 else max(
        timed, key=lambda kname: wev[-1][timed[kname]].elapsed_time(wev[-1][timed[kname] + 1]))
    jd = timed[dominant]

    # Timed region: K steps, right after the warmup, with events only around
    # the dominant kernel (the roofline's launch duration), so the step
    # clock carries as little instrumentation as possible.
    tev = event_rows(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(tev[s], marks=(jd, jd + 1))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    dominant_ms = float(np.mean([tev[s][jd].elapsed_time(tev[s][jd + 1]) for s in range(args.steps)]))

    n_pairs = int(B.schedule_views(p, sched)["desc"][0].item())

    # Per-kernel breakdown: K more steps with an event between every two kernels.
    events = event_rows(args.steps)
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    per_kernel = {n: float(np.mean([events[s][j].elapsed_time(events[s][j + 1])
                                    for s in range(args.steps)])) for j, n in enumerate(names)}
    per_kernel_median = {n: float(np.median([events[s][j].elapsed_time(events[s][j + 1])
                                             for s in range(args.steps)])) for j, n in enumerate(names)}

    # One cold step after a 512 MiB write has pushed the inputs out of the caches.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush.fill_(1)
    cold = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
    step(cold)
    torch.cuda.synchronize()
    cold_kernels = {n: cold[j].elapsed_time(cold[j + 1]) for j, n in enumerate(names)}
    cold_ms = cold[0].elapsed_time(cold[6])
    del flush

    # Secondary count: only the unmasked (query, key) entries of each tile
    # (the causal part of diagonal blocks and keys past a document end drop out).
    tm = B.schedule_views(p, sched)["task_meta"][:n_pairs].cpu().numpy().astype(np.int64)
    lens = np.diff(w.cu_seqlens.astype(np.int64))[tm[:, 4]]
    pos = tm[:, 2:3] + np.arange(8)[None, :]                       # query positions of the chunk
    valid_q = np.arange(8)[None, :] < tm[:, 3:4]
    seen = np.clip(np.minimum(pos, lens[:, None] - 1) - w.block * tm[:, 5:6] + 1, 0, w.block)
    unmasked_fraction = float((seen * valid_q).sum()) / (n_pairs * 8 * w.block) if n_pairs else 0.0

    fwd_f, bwd_f = pair_flops(w.block, w.head_dim)
    gemm = bwd_f // 5
    names_key = args.dq_mode + ("_b128" if args.block == 128 else "")
    value = n_pairs * (fwd_f + bwd_f) / (ms_step * 1e-3) / 1e12
    # useful contractions per pair done by each kernel
    pool = dq_mode in (B.DQ_ATOMIC_POOL, B.DQ_ATOMIC_POOL_BF16)
    useful = {"forward": fwd_f, "bwd_main": (5 if pool else 4) * gemm, "bwd_dq": (0 if pool else 1) * gemm}
    # Compulsory HBM bytes of each kernel (every tensor it must read or write
    # once), for the HBM-bound steps' GB/s against the 8 TB/s peak.
    T, hq, hkv, D = w.total_tokens, 16 * w.num_kv_heads, w.num_kv_heads, w.head_dim
    qb, kb = T * hq * D * 2, T * hkv * D * 2               # one bf16 [T, Hq, D] / [T, Hkv, D] tensor
    pool_bytes = {B.DQ_ATOMIC_POOL: 2 * qb, B.DQ_ATOMIC_POOL_BF16: qb}.get(dq_mode, 0)
    ds_bytes = n_pairs * 128 * w.block * 2 if dq_mode == B.DQ_DS_BUFFER else 0
    compulsory = {
        "forward": qb + 2 * kb + qb + T * hq * 4,
        "bwd_pre": 2 * qb + T * hq * 4 + 4 * kb + pool_bytes,
        "bwd_main": 2 * qb + 2 * kb + 2 * T * hq * 4 + 4 * kb + ds_bytes,
        "bwd_dq": ds_bytes + kb + qb if dq_mode == B.DQ_DS_BUFFER else (
            0 if pool else 2 * qb + 2 * kb + 2 * T * hq * 4 + qb),
        "bwd_post": 4 * kb + 2 * kb + (pool_bytes + qb if pool else 0),
    }
    gbps = {n: b / (per_kernel[n] * 1e-3) / 1e9 for n, b in compulsory.items() if b > 0 and per_kernel[n] > 0}
    tflops = {kname: n_pairs * f / (per_kernel[kname] * 1e-3) / 1e12 for kname, f in useful.items()
              if per_kernel[kname] > 0 and f > 0}
    bwd_ms = per_kernel["bwd_pre"] + per_kernel["bwd_main"] + per_kernel["bwd_dq"] + per_kernel["bwd_post"]
    bwd_tflops = n_pairs * bwd_f / (bwd_ms * 1e-3) / 1e12
    main_dq_ms = per_kernel["bwd_main"] + per_kernel["bwd_dq"]
    main_dq_tflops = n_pairs * bwd_f / (main_dq_ms * 1e-3) / 1e12 if main_dq_ms > 0 else 0.0
    dominant_tflops = n_pairs * useful[dominant] / (dominant_ms * 1e-3) / 1e12 if dominant_ms > 0 else 0.0

    traffic = measured_traffic(dominant, names_key)
    result = {
        "metric": "MSA fwd+bwd useful TFLOP/s and % of bf16 MFMA peak, 1xMI355X",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/k/v/dO, diagonal + uniform block selection)",
        "config": {"workload": f"{args.workload}: {len(w.cu_seqlens) - 1} document(s), T={w.total_tokens}, "
                               f"{w.num_kv_heads} KV heads x 16 query heads, D={w.head_dim}, "
                               f"key block {args.block}, chunk 8, top-k {w.topk}",
                   "selected_pairs": n_pairs, "num_cus": num_cus, "dq_mode": args.dq_mode,
                   "forward": args.forward},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "kernels_ms": {n: round(x, 4) for n, x in per_kernel.items()},
        "kernels_ms_median": {n: round(x, 4) for n, x in per_kernel_median.items()},
        "forward_plus_schedule_ms": round(per_kernel["schedule"] + per_kernel["forward"], 4),
        "backward_ms": round(bwd_ms, 4),
        "cold_step": {"ms": round(cold_ms, 4), "kernels_ms": {n: round(x, 4) for n, x in cold_kernels.items()},
                      "note": "one step after writing a 512 MiB buffer"},
        "unmasked_only": {"fraction_of_tile_entries": round(unmasked_fraction, 4),
                          "value": round(value * unmasked_fraction, 3), "unit": "TFLOP/s"},
        "kernels_useful_tflops": {n: round(x, 2) for n, x in tflops.items()},
        "kernels_pct_peak": {n: round(100.0 * x / PEAK_BF16_TFLOPS, 2) for n, x in tflops.items()},
        "kernels_compulsory_GBps": {n: round(x, 1) for n, x in gbps.items()},
        "kernels_pct_hbm_peak": {n: round(100.0 * x / PEAK_HBM_GBS, 1) for n, x in gbps.items()},
        "forward_pct_peak": round(100.0 * tflops["forward"] / PEAK_BF16_TFLOPS, 2),
        # the backward's five contractions per pair over the main and dQ kernels together
        "bwd_main_plus_dq": {"ms": round(per_kernel["bwd_main"] + per_kernel["bwd_dq"], 4),
                             "useful_tflops": round(main_dq_tflops, 2),
                             "pct_peak": round(100.0 * main_dq_tflops / PEAK_BF16_TFLOPS, 2)},
        "backward_useful_tflops": round(bwd_tflops, 2),
        "backward_pct_peak": round(100.0 * bwd_tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(dominant_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(dominant_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel": KERNEL_NAMES[names_key][dominant],
                     "launch_ms": round(dominant_ms, 4)},
    }
    if traffic is not None:
        # the measured HBM bytes of one launch over its duration: how close the
        # kernel's gathers run to the memory side's peak
        traffic_gbps = traffic / (dominant_ms * 1e-3) / 1e9
        result["roofline"]["traffic_GBps"] = round(traffic_gbps, 1)
        result["roofline"]["traffic_frac_hbm_peak"] = round(traffic_gbps / PEAK_HBM_GBS, 4)
    # The index scorer (the step that produces the selection; not part of the
    # timed step): same workload, synthetic index projections.
    from block_sparse_attention_k2q_amd.workloads import make_index_inputs
    qi, ki = (x.to(dev) for x in make_index_inputs(w))
    cu_dev = torch.from_numpy(w.cu_seqlens).to(dev)
    idx_scratch = torch.empty(B.msa_index_scratch_bytes(p), dtype=torch.uint8, device=dev)
    idx_sel = torch.empty(w.num_kv_heads, p.num_chunks, p.topk, dtype=torch.int32, device=dev)
    idx_ms = []
    for it in range(args.warmup + args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        B.msa_index_select(p, qi, ki, cu_dev, idx_scratch, idx_sel)
        b.record()
        if it >= args.warmup:
            idx_ms.append((a, b))
    torch.cuda.synchronize()
    idx_t = sorted(a.elapsed_time(b) for a, b in idx_ms)
    idx_bytes = 2 * qi.numel() * 2   # bf16 index queries and keys, read once
    result["index_scorer"] = {
        "ms_median": round(idx_t[len(idx_t) // 2], 4),
        "input_GBps": round(idx_bytes / (idx_t[len(idx_t) // 2] * 1e-3) / 1e9, 1),
        "note": "index scorer + top-k selection on the same workload (synthetic N(0,1) index "
                "projections, index dim 128); produces sel, outside the timed step"}
    del qi, ki, idx_scratch, idx_sel
    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = nbytes
    if not args.no_cpu_baseline:
        from oracle import msa_oracle as O
        sched_host = O.build_schedule(w.sel, w.cu_seqlens, w.block, num_cus)
        result["cpu_baseline"] = cpu_baseline(w, sched_host)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
