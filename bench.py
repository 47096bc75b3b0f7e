"""Benchmark of the fused attention forward on one MI355X.

One step = one fused forward (``fa_fwd``) over the whole batch of the headline
workload, B=1 H=32 N=8192 d=128, bf16 in, bf16 O + fp32 LSE out, inputs resident
in HBM before the timed region. Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline] [--unfused] [--launches-only]

The roofline entry is measured live: per-launch HIP events recorded on the stream
the kernel runs on, averaged over the timed region. Its ``traffic`` field comes
from the committed rocprofv3 counter summary of the same kernel
(profiles/fa_fwd_*_traffic.json) when its recorded source hash still matches the
kernel source, else null. The CPU baseline times the fp64 oracle on the host
cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6  # 256 CU x 4096 dense bf16 FLOP/clk x 2.4 GHz (AMD: "2.5 PFLOP/s")
HBM_PEAK_GBS = 8000.0
METRIC = "fwd attention TFLOP/s & % of bf16 MFMA peak, B=1 H=32 N=8192 d=128"
KERNEL_SRC = os.path.join(ROOT, "io_aware_softmax_attn_amd", "csrc", "fa_fwd.hip")


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, if still current."""
    path = os.path.join(ROOT, "profiles", f"fa_fwd_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, q, k, v, target_s: float = 10.0, max_heads: int = 32):
    """Time the fp64 oracle on whole heads of the workload until ``target_s`` of
    CPU work has accumulated (at least one head). Returns the dict for the JSON line."""
    import numpy as np  # noqa: F401  (BLAS threads are set before torch/numpy import in main)

    import attn_inputs
    from oracle import attention_fp64

    heads = 0
    t_total = 0.0
    flops = 0.0
    BH = w.B * w.H
    while heads < min(BH, max_heads) and t_total < target_s:
        b, h = divmod(heads, w.H)
        qh = attn_inputs.bf16_to_f64(q[b:b + 1, h:h + 1])
        kh = attn_inputs.bf16_to_f64(k[b:b + 1, h:h + 1])
        vh = attn_inputs.bf16_to_f64(v[b:b + 1, h:h + 1])
        t0 = time.perf_counter()
        attention_fp64(qh, kh, vh, w.scale)
        t_total += time.perf_counter() - t0
        flops += 4.0 * w.N * w.N * w.d
        heads += 1
    cores = len(os.sched_getaffinity(0))
    return {
        "value": flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{heads} of {BH} heads (all {w.N} query rows each), fp64 numpy two-pass oracle, "
                  f"{t_total:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true", help="time the three-kernel baseline instead")
    ap.add_argument("--launches-only", action="store_true",
                    help="only run warmup+steps launches (for profilers), print nothing but the JSON line")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the forward shards over heads with no exchange; see DESIGN.md).", file=sys.stderr)
        sys.exit(2)

    threads = str(len(os.sched_getaffinity(0)))
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ.setdefault(var, threads)

    import torch

    import attn_inputs
    import io_aware_softmax_attn_amd as fa

    w = attn_inputs.HEADLINE if args.workload is None else attn_inputs.WORKLOAD_BY_NAME[args.workload]
    q, k, v = attn_inputs.make_workload(w)
    dev = torch.device("cuda:0")
    qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qg)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    ws = None
    if args.unfused:
        ws = torch.empty(fa.fa_unfused_workspace_bytes(w.B, w.H, w.N), dtype=torch.uint8, device=dev)

    def launch():
        if args.unfused:
            fa.fa_unfused_fwd(qg, kg, vg, o, lse, ws, scale=w.scale, stream=stream)
        else:
            fa.fa_fwd(qg, kg, vg, o, lse, scale=w.scale, stream=stream)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        launch()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_ms = sum(per_launch_ms) / len(per_launch_ms)
    step_ms = max(wall * 1e3 / args.steps, avg_ms)

    tflops = w.flops / (avg_ms * 1e-3) / 1e12
    traffic = None if args.unfused else load_traffic(w.name)
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": False,
                   "path": "unfused-3-kernel" if args.unfused else "fused"},
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "kernel_ms_avg": round(avg_ms, 4),
            "kernel_ms_min": round(min(per_launch_ms), 4),
            "flops_per_launch": w.flops,
            "min_hbm_bytes_per_launch": w.min_hbm_bytes,
        },
    }
    if not args.launches_only and not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, q, k, v)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
