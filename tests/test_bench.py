"""bench.py end to end: on the GPU one short run prints one JSON line with
the fields the measurement needs (throughput, roofline of the dominant
kernel with its launch duration, per-kernel times and HBM rates); asked for
more than one GPU it refuses before touching any."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_json_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "kernels_ms",
                "kernels_compulsory_GBps"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1 and d["value"] > 0
    roof = d["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and 0 < roof["frac"] < 1
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["launch_ms"] > 0 and roof["kernel"].startswith("backward_kv_kernel")
    if roof["traffic"] is not None:   # the committed counter summary matches this kernel's source
        gbps = roof["traffic"] / (roof["launch_ms"] * 1e-3) / 1e9
        assert abs(roof["traffic_GBps"] - gbps) < 1.0 and 0 < roof["traffic_frac_hbm_peak"] < 1.5
    assert d["config"]["selected_pairs"] == 61696


def test_bench_refuses_several_gpus():
    # exits before touching a GPU, so it runs on the CPU too
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60, cwd=ROOT)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_cpu_baseline_shards_the_oracle_over_worker_processes():
    # the oracle's leg of the bench on the tiny workload, on the CPU: every
    # (index head, chunk) pair of it, one worker process per usable core
    import bench
    from block_sparse_attention_k2q_amd.workloads import make_workload
    from oracle import msa_oracle as O
    w = make_workload("tiny")
    s = O.build_schedule(w.sel, w.cu_seqlens, w.block, 256)
    r = bench.cpu_baseline(w, s)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0
    assert 1 <= r["cores"] <= len(os.sched_getaffinity(0))
    blocks = int((s["sel_clean"] >= 0).sum())
    assert r["sample"].startswith("all ") and f"({blocks} selected blocks)" in r["sample"]
