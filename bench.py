"""Benchmark of the fused attention forward on one MI355X.

One step = one fused forward (``fa_fwd``) over the whole batch of the headline
workload, B=1 H=32 N=8192 d=128, bf16 in, bf16 O + fp32 LSE out, inputs resident
in HBM before the timed region. Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline] [--unfused] [--launches-only]
  python bench.py --memory OUT_MD      (peak device memory, fused vs unfused)
  python bench.py --decode [--workload dec_...]   (decode-shaped forward, GB/s)
  python bench.py --backward [--workload NAME]    (backward dQ, dK, dV, TFLOP/s)
  python bench.py --all [--eager]      (one line per named forward workload)
  python bench.py --gemm [--shape M,N,K]          (context: a bf16 hipBLASLt GEMM)

The K timed launches of the fused forward are captured once in a HIP graph and
replayed between two HIP events on the stream they run on; the average launch
duration is the replay time over K. --eager launches them one by one from Python
instead, each between its own pair of events: that adds the event packets and the
dispatch latency to every launch (about 20 us, 2.5% at the benchmark workload)
and, for short launches, the host's per-call cost. The ``traffic`` field comes
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
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6  # 256 CU x 4096 dense bf16 FLOP/clk x 2.4 GHz (AMD: "2.5 PFLOP/s")
HBM_PEAK_GBS = 8000.0
METRIC = "fwd attention TFLOP/s & % of bf16 MFMA peak, B=1 H=32 N=8192 d=128"
KERNEL_SRC = os.path.join(ROOT, "io_aware_softmax_attn_amd", "csrc", "fa_fwd.hip")
UNFUSED_SRC = os.path.join(ROOT, "io_aware_softmax_attn_amd", "csrc", "fa_unfused.hip")
DECODE_SRC = os.path.join(ROOT, "io_aware_softmax_attn_amd", "csrc", "fa_decode.hip")


def metric_for(metric, shape):
    """The metric name with its trailing shape replaced by `shape` (the name as given
    when the shape is the one it is quoted on)."""
    return metric.rsplit(", ", 1)[0] + ", " + shape
DECODE_METRIC = "decode attention GB/s (Q, K, V read and O, LSE written once) & % of HBM peak, " \
                "B=16 H=32 Nq=1 Nk=8192 d=128"


def kernel_source_hash(path: str = KERNEL_SRC) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(workload: str, stem: str = "fa_fwd", src: str = KERNEL_SRC):
    """HBM bytes per launch from the committed counter summary, if still current."""
    path = os.path.join(ROOT, "profiles", f"{stem}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(src):
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


def _read_counter_csv(path):
    """(kernel name, counter name) -> list of per-dispatch values, in dispatch order."""
    import csv
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            key = (row["Kernel_Name"], row["Counter_Name"])
            out.setdefault(key, []).append((int(row["Dispatch_Id"]), float(row["Counter_Value"])))
    return {k: [v for _, v in sorted(vals)] for k, vals in out.items()}


UNFUSED_KERNELS = ("unf_qk_kernel", "unf_softmax_kernel", "unf_pv_kernel")


DECODE_KERNELS = ("dec_split_kernel", "dec_split_mfma_kernel", "dec_merge_kernel")
BWD_KERNELS = ("bwd_pre_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel", "bwd_dkdv_pair_kernel")
BWD_SRC = os.path.join(ROOT, "io_aware_softmax_attn_amd", "csrc", "fa_bwd.hip")


def summarize_pmc(fetch_csv, write_csv, workload, copy_bytes, unfused=False, decode=False, backward=False):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the fused kernel (or of the
    three unfused kernels, or of the two decode kernels, summed per launch) by what
    the same counters read for the plain copy of ``copy_bytes`` bytes in the same run."""
    import attn_inputs

    if decode:
        w = attn_inputs.DECODE_HEADLINE if workload is None else attn_inputs.DECODE_BY_NAME[workload]
    else:
        w = attn_inputs.HEADLINE if workload is None else attn_inputs.WORKLOAD_BY_NAME[workload]
    fetch = _read_counter_csv(fetch_csv)
    write = _read_counter_csv(write_csv)

    def pick(table, counter, pred):
        vals = [v for (k, c), vs in table.items() if c == counter and pred(k) for v in vs]
        if not vals:
            raise SystemExit(f"no {counter} values for the requested kernel in the CSV")
        return vals

    def per_launch(table, counter):
        """Average KiB per launch: one kernel (fused) or the sum of the three."""
        names = (DECODE_KERNELS if decode else BWD_KERNELS if backward else UNFUSED_KERNELS if unfused
                 else ("fa_fwd_kernel",))
        # the decode split runs one of two kernels, by the number of query rows
        names = [n for n in names if any(n in k for (k, c) in table if c == counter)]
        total, raw = 0.0, []
        for name in names:
            vals = pick(table, counter, lambda k, n=name: n in k)
            total += sum(vals) / len(vals)
            raw.append(vals)
        per = [round(sum(r[i] for r in raw), 1) for i in range(min(len(r) for r in raw))]
        return total, per

    is_copy = lambda k: "fa_fwd_kernel" not in k and "unf_" not in k and "dec_" not in k and "bwd_" not in k
    copy_fetch = pick(fetch, "FETCH_SIZE", is_copy)[0] * 1024.0
    copy_write = pick(write, "WRITE_SIZE", is_copy)[0] * 1024.0
    f_scale = copy_bytes / copy_fetch
    w_scale = copy_bytes / copy_write
    fa_fetch_kib, fa_fetch = per_launch(fetch, "FETCH_SIZE")
    fa_write_kib, fa_write = per_launch(write, "WRITE_SIZE")
    fetch_b = fa_fetch_kib * 1024.0 * f_scale
    write_b = fa_write_kib * 1024.0 * w_scale
    rec = {
        "workload": w.name,
        "path": ("decode split+merge" if decode else "backward" if backward else "unfused-3-kernel" if unfused
                 else "fused"),
        "kernel_source_sha256_16": kernel_source_hash(DECODE_SRC if decode else BWD_SRC if backward
                                                      else UNFUSED_SRC if unfused else KERNEL_SRC),
        "hbm_bytes_per_launch": round(fetch_b + write_b),
        "fetch_bytes_per_launch": round(fetch_b),
        "write_bytes_per_launch": round(write_b),
        "min_hbm_bytes_per_launch": w.min_hbm_bytes,
        "ratio_to_min": round((fetch_b + write_b) / w.min_hbm_bytes, 4),
        "copy_calibration_bytes": copy_bytes,
        "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4),
        "fetch_kib_raw_per_launch": fa_fetch,
        "write_kib_raw_per_launch": fa_write,
        "commands": [f"rocprofv3 --pmc {ctr} -d <out>/pmc_{w.name}_{ctr} -o c --output-format csv -- python3 bench.py "
                     + ("--decode " if decode else "--backward " if backward else "--unfused " if unfused else "")
                     + f"--workload {w.name} --launches-only --steps 2 --warmup 1 --copy-calibration {copy_bytes}"
                     for ctr in ("FETCH_SIZE", "WRITE_SIZE")],
    }
    stem = "fa_decode" if decode else "fa_bwd" if backward else "fa_unfused" if unfused else "fa_fwd"
    if backward:  # algorithmic bytes: read q, k, v, o, dO and lse, write dq, dk, dv
        rec["min_hbm_bytes_per_launch"] = w.B * w.H * w.N * (16 * w.d + 4)
        rec["ratio_to_min"] = round((fetch_b + write_b) / rec["min_hbm_bytes_per_launch"], 4)
    path = os.path.join(ROOT, "profiles", f"{stem}_{w.name}_traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


IO_SWEEP_ORDERS = (0, 1, 2)
IO_SWEEP_LENGTHS = (2048, 4096, 8192, 16384)
IO_SWEEP_SHAPE = (1, 32, 128)  # B, H, d
IO_SWEEP_CMD = ("rocprofv3 --pmc {ctr} -d {dir}/pmc_o{order}_n{n}_{ctr} -o c --output-format csv -- "
                "python3 bench.py --shape {B},{H},{n},{d} --tile-order {order} --br 256 --steps 2 --warmup 1 "
                "--launches-only --copy-calibration 1073741824")
# The 128-row query tile (fa_fwd_blocks), XCD-aware order: twice the query tiles per
# head, so twice the K/V passes that the on-chip caches must absorb.
IO_SWEEP_BR_CMD = ("rocprofv3 --pmc {ctr} -d {dir}/pmc_b128_n{n}_{ctr} -o c --output-format csv -- "
                   "python3 bench.py --shape {B},{H},{n},{d} --br 128 --steps 2 --warmup 1 "
                   "--launches-only --copy-calibration 1073741824")


def summarize_io_sweep(sweep_dir, copy_bytes):
    """HBM traffic of the fused kernel per workgroup-to-tile order and sequence
    length, from FETCH_SIZE / WRITE_SIZE runs made with IO_SWEEP_CMD, written to
    profiles/fa_fwd_io_sweep.md next to two models: every byte once, and every
    query tile re-reading its head's K and V."""
    B, H, d = IO_SWEEP_SHAPE
    names = {0: "XCD-aware", 1: "dispatch order", 2: "query-tile-major"}
    rows = []
    runs = [(order, 256, f"pmc_o{order}_n{{n}}") for order in IO_SWEEP_ORDERS]
    if os.path.isdir(os.path.join(sweep_dir, f"pmc_b128_n{IO_SWEEP_LENGTHS[0]}_FETCH_SIZE")):
        runs.append((0, 128, "pmc_b128_n{n}"))
    for order, br, stem in runs:
        for n in IO_SWEEP_LENGTHS:
            vals = {}
            for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
                table = _read_counter_csv(os.path.join(sweep_dir, stem.format(n=n) + f"_{ctr}",
                                                       "c_counter_collection.csv"))
                fa_vals = [v for (kname, c), vs in table.items() if c == ctr and "fa_fwd_kernel" in kname for v in vs]
                copy = [v for (kname, c), vs in table.items() if c == ctr and "fa_fwd_kernel" not in kname for v in vs]
                vals[ctr] = sum(fa_vals) / len(fa_vals) * copy_bytes / copy[0]
            total = vals["FETCH_SIZE"] + vals["WRITE_SIZE"]
            minimum = B * H * n * (8 * d + 4)
            tiles = -(-n // br)
            reread = B * H * (tiles * 4 * n * d + n * (4 * d + 4))  # K, V per query tile; Q, O, LSE once
            rows.append((order, br, n, total, minimum, reread))
    lines = [
        "# Fused-kernel HBM traffic by workgroup-to-tile order and sequence length",
        "",
        f"B={B} H={H} d={d}; BR query rows per workgroup (256 unless stated). Bytes per launch from "
        "FETCH_SIZE + WRITE_SIZE (KiB per dispatch), each scaled by what the counter reads for a 1 GiB "
        "device-to-device copy in the same run, averaged over the 3 launches of each run. One run per order "
        "(or BR), length and counter:",
        "",
        "```",
        IO_SWEEP_CMD.format(ctr="<FETCH_SIZE|WRITE_SIZE>", dir=sweep_dir.rstrip("/"), order="<order>", n="<N>",
                            B=B, H=H, d=d),
        IO_SWEEP_BR_CMD.format(ctr="<FETCH_SIZE|WRITE_SIZE>", dir=sweep_dir.rstrip("/"), n="<N>", B=B, H=H, d=d),
        "```",
        "",
        "Models: `once` = B*H*N*(8d+4) (Q, K, V read once, O and LSE written once); `re-read` = K and V "
        "read again by every query tile of their head, ceil(N/BR) times, plus Q, O, LSE once.",
        "",
        "| order | BR | N | bytes per launch | / once | / re-read |",
        "|---|---|---|---|---|---|",
    ]
    for order, br, n, total, minimum, reread in rows:
        lines.append(f"| {order} {names[order]} | {br} | {n} | {total:,.0f} | {total / minimum:.3f} | "
                     f"{total / reread:.3f} |")
    lines += ["", f"Kernel source sha256[:16] of fa_fwd.hip: {kernel_source_hash()}."]
    path = os.path.join(ROOT, "profiles", "fa_fwd_io_sweep.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_parity(jsonl, command, out_md="profiles/parity_gpu.md"):
    """No GPU work: turn the raw error records the GPU parity tests append to
    FA_PARITY_RECORD (one JSON object per case) into a table, and copy the records
    next to it (profiles/parity_gpu.jsonl)."""
    recs = [json.loads(line) for line in open(jsonl) if line.strip()]
    out_md = os.path.join(ROOT, out_md)
    with open(os.path.splitext(out_md)[0] + ".jsonl", "w") as f:
        for r in recs:
            f.write(json.dumps(r) + "\n")

    def g(x, fmt="{:.3e}"):
        return "-" if x is None else fmt.format(x)

    lines = [
        "# GPU parity against the fp64 oracle (raw figures)",
        "",
        f"Command: `{command}`",
        "",
        "Gates: max|dO| <= 1e-2 on every element with |O| < 2; from |O| = 2 on, max(|dO| - half bf16 ulp) "
        "<= 1e-2 (the output rounding alone is up to 0.0078 there); max|dLSE| <= 1e-3; max|dO| <= 2 x E_unf, "
        "the error of the bf16 unfused computation on the same rows. `n > 1e-2` counts elements whose raw "
        "|dO| exceeds 1e-2.",
        "",
        "## Forward (fused, both query-tile heights), unfused baseline, decode",
        "",
        r"| path | case | BR | rows | max\|O_ref\| | max\|dO\| | max\|dO\| (\|O\|<2) | beyond half-ulp (\|O\|>=2) "
        r"| n > 1e-2 / elements | max\|dLSE\| | E_unf | max\|dO\| / E_unf |",
        "|---|---|---|---|---|---|---|---|---|---|---|---|",
    ]
    for r in recs:
        if r["kind"].startswith("backward"):
            continue
        ratio = r["max_dO"] / r["E_unf"] if r.get("E_unf") else None
        lines.append(f"| {r['kind']} | {r['case']} | {r.get('br', '-')} | {r['rows_checked']} | "
                     f"{r['max_abs_O_ref']:.3f} | {g(r['max_dO'])} | {g(r['max_dO_narrow'])} | "
                     f"{g(r['max_dO_wide_beyond_rounding'])} | {r['n_over_tol']} / {r['n_elements']} | "
                     f"{g(r['max_dLSE'])} | {g(r.get('E_unf'))} | {g(ratio, '{:.2f}')} |")
    bw = [r for r in recs if r["kind"].startswith("backward")]
    if bw:
        lines += ["", "## Backward (gate: each gradient's max error <= 2 x the bf16 unfused backward's)", "",
                  "| case | dQ | 2 E_unf(dQ) | dK | 2 E_unf(dK) | dV | 2 E_unf(dV) |", "|---|---|---|---|---|---|---|"]
        for r in bw:
            lines.append(f"| {r['case']} | " + " | ".join(
                f"{g(r['max_d' + n])} | {g(2 * r['E_unf_' + n])}" for n in ("dQ", "dK", "dV")) + " |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out_md)


def summarize_trace(stats_csv, command, workload, steps=50, bench_json=None):
    """Write the per-kernel duration summary of a rocprofv3 --stats run, with the
    command that produced it and the algorithmic rate at the average duration. With
    bench_json (the JSON line of a bench.py run made in the same GPU session), quote
    that line's rate and step time next to the trace."""
    import csv

    import attn_inputs

    rows = list(csv.DictReader(open(stats_csv)))
    backward = any("bwd_dq_kernel" in r["Name"] for r in rows)
    fused = not backward and any("fa_fwd_kernel" in r["Name"] for r in rows)
    decode = any("dec_split" in r["Name"] for r in rows)
    if decode:
        w = attn_inputs.DECODE_HEADLINE if workload is None else attn_inputs.DECODE_BY_NAME[workload]
        shape = f"B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} d={w.d}"
    else:
        w = attn_inputs.HEADLINE if workload is None else attn_inputs.WORKLOAD_BY_NAME[workload]
        shape = f"B={w.B} H={w.H} N={w.N} d={w.d}"
    lines = [f"# Kernel durations, workload {w.name} ({shape})", "",
             "Command, run from the repository root with TMPDIR=/tmp:", "", "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us | stddev us |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        short = name[:60]
        for base in ("fa_fwd_kernel", "unf_qk_kernel", "unf_softmax_kernel", "unf_pv_kernel") + DECODE_KERNELS + \
                BWD_KERNELS:
            if base in name:
                args = re.findall(r"ILi(\d+)E(?:Li(\d+)E)?", name)
                if args:
                    short = f"{base}<{','.join(x for x in args[0] if x)}>"
                else:
                    dim = next((dd for dd in ("128", "64") if f"<{dd}>" in name), None)
                    short = f"{base}<{dim}>" if dim else base
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['StdDev']) / 1e3:.1f} |")
    if fused:
        r = next(r for r in rows if "fa_fwd_kernel" in r["Name"])
        avg_s = float(r["AverageNs"]) * 1e-9
        tf = w.flops / avg_s / 1e12
        lines += ["", f"Fused kernel at its average duration: {w.flops:.4e} FLOP per launch -> {tf:.1f} TFLOP/s, "
                      f"{tf / MFMA_BF16_PEAK_TFLOPS:.4f} of the {MFMA_BF16_PEAK_TFLOPS} TFLOP/s bf16 MFMA peak "
                      "(the average over every launch, warmup included)."]
        # The per-dispatch trace next to the stats file: the last `steps` launches are
        # the timed region, the span that bench.py's own events measure.
        trace_csv = stats_csv.replace("kernel_stats", "kernel_trace")
        if trace_csv != stats_csv and os.path.exists(trace_csv):
            disp = sorted((t for t in csv.DictReader(open(trace_csv)) if "fa_fwd_kernel" in t["Kernel_Name"]),
                          key=lambda t: int(t["Start_Timestamp"]))[-steps:]
            durs = [(int(t["End_Timestamp"]) - int(t["Start_Timestamp"])) * 1e-3 for t in disp]
            gaps = [(int(b["Start_Timestamp"]) - int(a["End_Timestamp"])) * 1e-3 for a, b in zip(disp, disp[1:])]
            mean = sum(durs) / len(durs)
            lines.append(f"The last {len(disp)} launches (the timed region): {mean:.1f} us per kernel on average "
                         f"(min {min(durs):.1f}, max {max(durs):.1f}), {sum(gaps) / max(len(gaps), 1):.2f} us "
                         f"between kernels on average -> {w.flops / (mean * 1e-6) / 1e12:.1f} TFLOP/s.")
        lines.append(f"Kernel source sha256[:16] of fa_fwd.hip: {kernel_source_hash()}.")
    if decode:
        split = [r for r in rows if any(kname in r["Name"] for kname in DECODE_KERNELS)]
        total_s = sum(float(r["AverageNs"]) for r in split) * 1e-9
        gbs = w.min_hbm_bytes / total_s / 1e9
        lines += ["", f"Decode kernels (split + merge) at their average durations: {w.min_hbm_bytes} algorithmic "
                      f"HBM bytes per call -> {gbs:.0f} GB/s, {gbs / HBM_PEAK_GBS:.4f} of the {HBM_PEAK_GBS:.0f} GB/s "
                      f"HBM peak.",
                  f"Kernel source sha256[:16] of fa_decode.hip: {kernel_source_hash(DECODE_SRC)}."]
    if backward:
        bwd = [r for r in rows if any(kname in r["Name"] for kname in BWD_KERNELS)]
        total_s = sum(float(r["AverageNs"]) for r in bwd) * 1e-9
        tf = 2.5 * w.flops / total_s / 1e12
        lines += ["", f"Backward kernels (pre + dq + dkdv) at their average durations: {2.5 * w.flops:.4e} FLOP "
                      f"(10*B*H*N^2*d) per call -> {tf:.1f} TFLOP/s, {tf / MFMA_BF16_PEAK_TFLOPS:.4f} of the "
                      f"{MFMA_BF16_PEAK_TFLOPS} TFLOP/s bf16 MFMA peak. The forward launch in the table makes O and "
                      f"LSE for the backward's inputs.",
                  f"Kernel source sha256[:16] of fa_bwd.hip: {kernel_source_hash(BWD_SRC)}."]
    if bench_json:
        with open(bench_json) as f:
            rec = json.loads(f.read().strip().splitlines()[-1])
        r = rec["roofline"]
        cmd = f"python3 bench.py --gpus {rec['n_gpus']} --steps {rec['steps']} --warmup {rec['warmup']}"
        if rec["config"].get("workload") != attn_inputs.HEADLINE.name:
            cmd += f" --workload {rec['config']['workload']} --no-cpu-baseline"
        lines += ["", f"`{cmd}`, run just before the trace in the same GPU session: {rec['value']} {rec['unit']} "
                      f"({r['frac']} of peak), ms_per_step {rec['ms_per_step']}; per launch {r['kernel_ms_avg']} ms "
                      f"on average over the {rec['steps']} timed launches (median {r.get('kernel_ms_median')}, "
                      f"min {r.get('kernel_ms_min')}, max {r.get('kernel_ms_max')} over {r.get('timing_samples')} "
                      f"samples, each {r.get('timing_sample')})."]
    stem = "fa_fwd" if fused else "fa_decode" if decode else "fa_bwd" if backward else "fa_unfused"
    path = os.path.join(ROOT, "profiles", f"{stem}_{w.name}_kernel_trace.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


SQ_COUNTERS = ("SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
               "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_INSTS_LDS")


def summarize_counters(counter_csv, command, workload):
    """Matrix-core occupancy and instruction mix of each kernel in a rocprofv3 --pmc
    run of SQ_COUNTERS, averaged over its dispatches after the first.
    SQ_BUSY_CYCLES sums over the 32 shader engines and SQ_VALU_MFMA_BUSY_CYCLES over
    the 1024 SIMDs, so busy = MFMA / (BUSY / 32 * 1024)."""
    import collections
    import csv

    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in csv.DictReader(open(counter_csv)):
        key = int(r["Dispatch_Id"])
        per[key][r["Counter_Name"]] += float(r["Counter_Value"])
        names[key] = r["Kernel_Name"]
    kernels = collections.defaultdict(list)
    for key in sorted(per):
        base = re.sub(r"\(.*", "", names[key])
        kernels[base].append(per[key])
    lines = [f"# SQ counters, workload {workload}", "", "Command, run from the repository root with TMPDIR=/tmp:", "",
             "```", command, "```", "",
             "| kernel | dispatches | MFMA busy | VALU insts / MFMA insts | LDS insts / MFMA insts | "
             "VALU-MFMA co-issue / MFMA busy | waves waiting on a dependency | kernel cycles |",
             "|---|---|---|---|---|---|---|---|"]
    for base, ds in kernels.items():
        if not any(x in base for x in ("fa_fwd_kernel", "dec_", "bwd_", "unf_")):
            continue
        use = ds[1:] if len(ds) > 1 else ds
        c = {n: sum(d.get(n, 0.0) for d in use) / len(use) for n in SQ_COUNTERS}
        busy = c["SQ_BUSY_CYCLES"] / 32.0
        mf = c["SQ_VALU_MFMA_BUSY_CYCLES"]
        m = re.search(r"\d+([a-z_]+_kernel)((?:ILi\d+E)*(?:Li\d+E)*)", base)
        short = (m.group(1) + "<" + ",".join(re.findall(r"Li(\d+)E", m.group(2))) + ">") if m else base[:60]
        lines.append(f"| `{short}` | {len(use)} | {mf / (busy * 1024):.3f} | "
                     f"{c['SQ_INSTS_VALU'] / max(c['SQ_INSTS_MFMA'], 1):.2f} | "
                     f"{c['SQ_INSTS_LDS'] / max(c['SQ_INSTS_MFMA'], 1):.2f} | "
                     f"{c['SQ_VALU_MFMA_COEXEC_CYCLES'] / max(mf, 1):.2f} | "
                     f"{c['SQ_WAIT_INST_ANY'] / max(c['SQ_WAVE_CYCLES'], 1):.2f} | {busy:.4g} |")
    # a backward run also launches the forward that makes its O and LSE
    stem = "fa_bwd" if any("bwd_" in b for b in kernels) else "fa_decode" if any(
        "dec_" in b for b in kernels) else "fa_fwd"
    path = os.path.join(ROOT, "profiles", f"{stem}_{workload}_counters.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def decode_cpu_baseline(w, q, k, v, target_s: float = 10.0):
    """The fp64 oracle on whole heads of the decode workload until ``target_s`` of CPU
    work has accumulated; rate in algorithmic GB/s like the GPU figure."""
    import attn_inputs
    from oracle import attention_fp64

    heads, t_total = 0, 0.0
    BH = w.B * w.H
    while heads < BH and t_total < target_s:
        b, h = divmod(heads, w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        qh, kh, vh = (attn_inputs.bf16_to_f64(t[sl]) for t in (q, k, v))
        t0 = time.perf_counter()
        attention_fp64(qh, kh, vh, w.scale)
        t_total += time.perf_counter() - t0
        heads += 1
    per_head = w.min_hbm_bytes / BH
    return {
        "value": heads * per_head / t_total / 1e9,
        "unit": "GB/s",
        "cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"{heads} of {BH} heads (all {w.Nq} query rows against {w.Nk} keys each), fp64 numpy "
                  f"two-pass oracle, {t_total:.1f} s",
    }


def graph_chunks(steps: int) -> int:
    """Number of equal graph replays the `steps` timed launches are split into (up to
    five, the largest that divides `steps`), so that the timing has a spread."""
    for r in (5, 4, 3, 2):
        if steps % r == 0:
            return r
    return 1


def time_launches(torch, launch, steps, stream, use_graph):
    """Run exactly `steps` timed launches of `launch(stream)` and return (per-launch ms
    list, wall seconds). With use_graph, steps/R launches are captured once in a HIP
    graph (launched on torch's capture stream; R = graph_chunks(steps)) and replayed
    R times untimed (the first replay also uploads the graph; together they run the
    same `steps` launches untimed as a single graph of all of them would), then R
    times more, each replay between two events on `stream`: the list holds each
    replay's time over its launch count. Otherwise each launch is issued eagerly
    between its own pair of events."""
    if use_graph:
        r = graph_chunks(steps)
        per = steps // r
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per):
                launch(None)  # torch's current stream is the capture stream here
        for _ in range(r):
            g.replay()
        torch.cuda.synchronize()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(r)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(r)]
        t0 = time.perf_counter()
        for i in range(r):
            starts[i].record(stream)
            g.replay()
            ends[i].record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) / per for a, b in zip(starts, ends)], time.perf_counter() - t0
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        launch(stream)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [a.elapsed_time(b) for a, b in zip(starts, ends)], wall


def timing_stats(per_ms, use_graph, steps):
    """Spread of the per-launch times: one sample per graph replay (its time over its
    launch count) or per eager launch."""
    xs = sorted(per_ms)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    return {"kernel_ms_median": round(med, 4), "kernel_ms_min": round(xs[0], 4), "kernel_ms_max": round(xs[-1], 4),
            "timing_samples": n,
            "timing_sample": (f"one graph replay of {steps // n} launches" if use_graph else "one launch")}


def decode_bench(args):
    """Time the decode-shaped forward (split + merge kernels) and print one JSON line."""
    import torch

    import attn_inputs
    import io_aware_softmax_attn_amd as fa

    if args.shape:
        B, H, Nq, Nk, d = (int(x) for x in args.shape.split(","))
        w = attn_inputs.DecodeWorkload(f"dec_b{B}h{H}_q{Nq}_k{Nk}_d{d}", B, H, Nq, Nk, d, seed=0)
    else:
        w = attn_inputs.DECODE_HEADLINE if args.workload is None else attn_inputs.DECODE_BY_NAME[args.workload]
    q, k, v = attn_inputs.make_decode_workload(w)
    dev = torch.device("cuda:0")
    qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qg)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    splits, chunk, ws_bytes = fa.fa_decode_plan(w.B, w.H, w.Nq, w.Nk, w.d)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # K and V of the benchmark shape (2.1 GB) exceed the 256 MB Infinity Cache many
    # times over, so back-to-back calls cannot serve each other from cache.
    for _ in range(args.warmup):
        fa.fa_decode_fwd(qg, kg, vg, o, lse, ws, scale=w.scale, stream=stream)
    torch.cuda.synchronize()
    use_graph = not (args.eager or args.launches_only)
    per_ms, wall = time_launches(
        torch, lambda s: fa.fa_decode_fwd(qg, kg, vg, o, lse, ws, scale=w.scale, stream=s), args.steps, stream,
        use_graph)
    avg_ms = sum(per_ms) / len(per_ms)
    gbs = w.min_hbm_bytes / (avg_ms * 1e-3) / 1e9
    line = {
        "metric": metric_for(DECODE_METRIC, f"B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} d={w.d}"),
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(max(wall * 1e3 / args.steps, avg_ms), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "splits": splits, "chunk": chunk, "path": "decode split+merge",
                   "launch": "graph" if use_graph else "eager"},
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": load_traffic(w.name, "fa_decode", DECODE_SRC),
            "kernel_ms_avg": round(avg_ms, 4),
            **timing_stats(per_ms, use_graph, args.steps),
            "min_hbm_bytes_per_launch": w.min_hbm_bytes,
            "tflops": round(w.flops / (avg_ms * 1e-3) / 1e12, 2),
        },
    }
    if not args.launches_only and not args.no_cpu_baseline:
        line["cpu_baseline"] = decode_cpu_baseline(w, q, k, v)
    print(json.dumps(line), flush=True)


BWD_METRIC = "bwd attention TFLOP/s (10*B*H*N^2*d) & % of bf16 MFMA peak, B=1 H=32 N=8192 d=128"


def backward_bench(args):
    """Time the backward (three kernels) on a prefill workload and print one JSON line.
    Algorithmic FLOPs: the five N x N x d products of the backward, 10*B*H*N^2*d
    (2.5x the forward's four), whatever the kernels recompute."""
    import torch

    import attn_inputs
    import io_aware_softmax_attn_amd as fa

    if args.shape:
        B, H, N, d = (int(x) for x in args.shape.split(","))
        w = attn_inputs.Workload(f"b{B}h{H}_n{N}_d{d}", B, H, N, d, seed=0)
    else:
        w = attn_inputs.HEADLINE if args.workload is None else attn_inputs.WORKLOAD_BY_NAME[args.workload]
    q, k, v = attn_inputs.make_workload(w)
    g = torch.Generator().manual_seed(w.seed + 7919)
    dO = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    dev = torch.device("cuda:0")
    qg, kg, vg, gg = (t.to(dev) for t in (q, k, v, dO))
    o, lse = fa.forward(qg, kg, vg, scale=w.scale)
    dq, dk, dv = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.N), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        fa.fa_bwd(qg, kg, vg, o, lse, gg, dq, dk, dv, ws, scale=w.scale, stream=stream)
    torch.cuda.synchronize()
    use_graph = not (args.eager or args.launches_only)
    per_ms, wall = time_launches(
        torch, lambda s: fa.fa_bwd(qg, kg, vg, o, lse, gg, dq, dk, dv, ws, scale=w.scale, stream=s), args.steps,
        stream, use_graph)
    avg_ms = sum(per_ms) / len(per_ms)
    flops = 2.5 * w.flops
    tf = flops / (avg_ms * 1e-3) / 1e12
    traffic = load_traffic(w.name, "fa_bwd", BWD_SRC)
    line = {
        "metric": metric_for(BWD_METRIC, f"B={w.B} H={w.H} N={w.N} d={w.d}"),
        "value": round(tf, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(max(wall * 1e3 / args.steps, avg_ms), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": False, "path": "backward",
                   "launch": "graph" if use_graph else "eager"},
        "roofline": {
            "bound": "mfma",
            "achieved": round(tf, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "kernel_ms_avg": round(avg_ms, 4),
            **timing_stats(per_ms, use_graph, args.steps),
            "flops_per_launch": flops,
            "executed_flops_per_launch": 3.5 * w.flops,
            # read q, k, v, o, dO and lse once, write dq, dk and dv once
            "min_hbm_bytes_per_launch": w.B * w.H * w.N * (16 * w.d + 4),
            "hbm_gb_per_s": None if traffic is None else round(traffic / (avg_ms * 1e-3) / 1e9, 1),
            "hbm_frac_of_peak": None if traffic is None else round(traffic / (avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        },
    }
    if not args.launches_only and not args.no_cpu_baseline:
        from oracle import attention_backward_fp64

        heads, t_total = 0, 0.0
        while heads < w.B * w.H and t_total < 10.0:
            b, h = divmod(heads, w.H)
            sl = (slice(b, b + 1), slice(h, h + 1))
            args_h = [attn_inputs.bf16_to_f64(t[sl]) for t in (q, k, v, dO)]
            t1 = time.perf_counter()
            attention_backward_fp64(*args_h, w.scale)
            t_total += time.perf_counter() - t1
            heads += 1
        line["cpu_baseline"] = {
            "value": heads * 10.0 * w.N * w.N * w.d / t_total / 1e12,
            "unit": "TFLOP/s",
            "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} heads (all {w.N} rows each), fp64 numpy backward oracle, "
                      f"{t_total:.1f} s",
        }
    print(json.dumps(line), flush=True)


# Shapes of the device-memory comparison: (B, H, d, sequence lengths).
MEMORY_SHAPES = ((2, 16, 128, (1024, 2048, 4096, 8192)), (4, 16, 64, (1024, 2048, 4096, 8192)))


def gemm_bench(args):
    """Time a dense bf16 matrix product C = A B (torch.mm, which ROCm serves from
    hipBLASLt), by default M = N = K = 8192: 2*8192^3 FLOP, the same count as one
    forward launch at B=1 H=32 N=8192 d=128. Context only, not the product: the rate
    a vendor-tuned contraction sustains on this part under the same power limit,
    against the same 2.4 GHz peak. Timed like the forward (graph replays)."""
    import torch

    M, N, K = (int(x) for x in (args.shape or "8192,8192,8192").split(","))
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(0)
    a = torch.randn((M, K), generator=g).to(torch.bfloat16).to(dev).contiguous()
    b = torch.randn((K, N), generator=g).to(torch.bfloat16).to(dev).contiguous()
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def launch(s=stream):
        torch.mm(a, b, out=c)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    use_graph = not (args.eager or args.launches_only)
    per_ms, _ = time_launches(torch, launch, args.steps, stream, use_graph)
    avg_ms = sum(per_ms) / len(per_ms)
    flops = 2.0 * M * N * K
    tflops = flops / (avg_ms * 1e-3) / 1e12
    line = {"metric": f"bf16 GEMM TFLOP/s (context), M={M} N={N} K={K}", "value": round(tflops, 2),
            "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
            "config": {"op": "torch.mm", "M": M, "N": N, "K": K, "launch": "graph" if use_graph else "eager"},
            "frac_of_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "kernel_ms_avg": round(avg_ms, 4),
            **timing_stats(per_ms, use_graph, args.steps)}
    print(json.dumps(line), flush=True)


def footprint_bytes(B: int, H: int, N: int, d: int, fused: bool) -> int:
    """Device bytes one forward holds at its peak: Q, K, V and O (bf16) and LSE
    (fp32), plus, on the unfused path, the score matrix S (fp32) and the
    probabilities P (bf16) of every head. The fused footprint grows with N, the
    unfused one with N^2 ("01 · 注意力为什么是 IO 瓶颈", section 6: the memory saved
    at 2K and 4K sequence length, growing linearly with it)."""
    base = B * H * N * (8 * d + 4)
    return base if fused else base + 6 * B * H * N * N


def memory_comparison(out_md: str, command: str):
    """Peak device memory of one fused and one unfused forward per shape, measured
    with torch's allocator statistics (the library itself allocates nothing; O, LSE
    and the unfused workspace come from torch), next to footprint_bytes."""
    import torch

    import attn_inputs
    import io_aware_softmax_attn_amd as fa

    dev = torch.device("cuda:0")
    recs = []
    for B, H, d, lengths in MEMORY_SHAPES:
        for N in lengths:
            q, k, v = (t.to(dev) for t in attn_inputs.make_qkv(B, H, N, d, seed=N))
            rec = {"B": B, "H": H, "N": N, "d": d}
            for path, fn in (("fused", fa.forward), ("unfused", fa.unfused_forward)):
                torch.cuda.synchronize()
                torch.cuda.empty_cache()
                torch.cuda.reset_peak_memory_stats(dev)
                outs = fn(q, k, v)
                torch.cuda.synchronize()
                # Requested bytes: the tensors' own sizes, before the allocator rounds
                # them to its blocks (the rounded peak is kept for reference).
                rec[f"{path}_peak_bytes"] = torch.cuda.memory_stats(dev)["requested_bytes.all.peak"]
                rec[f"{path}_peak_block_bytes"] = torch.cuda.max_memory_allocated(dev)
                rec[f"{path}_model_bytes"] = footprint_bytes(B, H, N, d, path == "fused")
                del outs
            rec["ratio"] = rec["unfused_peak_bytes"] / rec["fused_peak_bytes"]
            del q, k, v
            recs.append(rec)
            print(json.dumps(rec), flush=True)
    lines = [
        "# Peak device memory of one forward, fused vs unfused",
        "",
        "Command, run from the repository root:",
        "",
        "```",
        command,
        "```",
        "",
        "Peak requested bytes from torch.cuda.memory_stats around one call, with Q, K and V already resident. "
        "The model column is B*H*N*(8d+4) for the fused path (Q, K, V, O, LSE) plus 6*B*H*N^2 for the "
        "unfused path's S (fp32) and P (bf16).",
        "",
        "| B | H | N | d | fused MiB | unfused MiB | unfused / fused | both equal the model |",
        "|---|---|---|---|---|---|---|---|",
    ]
    for r in recs:
        ok = r["fused_peak_bytes"] == r["fused_model_bytes"] and r["unfused_peak_bytes"] == r["unfused_model_bytes"]
        lines.append(f"| {r['B']} | {r['H']} | {r['N']} | {r['d']} | {r['fused_peak_bytes'] / 2**20:.1f} | "
                     f"{r['unfused_peak_bytes'] / 2**20:.1f} | {r['ratio']:.1f}x | {'yes' if ok else 'no'} |")
    os.makedirs(os.path.dirname(os.path.abspath(out_md)), exist_ok=True)
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return recs


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
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="first run one plain device-to-device copy of BYTES bytes (a known-size reference "
                         "dispatch for the FETCH_SIZE/WRITE_SIZE counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: read two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) of a --copy-calibration run and write profiles/fa_fwd_<workload>_traffic.json")
    ap.add_argument("--summarize-trace", nargs="+", metavar="STATS_CSV COMMAND [BENCH_JSON]",
                    help="no GPU work: turn a rocprofv3 --kernel-trace --stats kernel_stats.csv into "
                         "profiles/<kernel>_<workload>_kernel_trace.md, recording COMMAND as its origin, and "
                         "quoting the bench.py JSON line of the same GPU session when given")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("COUNTER_CSV", "COMMAND"),
                    help="no GPU work: turn a rocprofv3 --pmc counter_collection.csv of SQ counters into "
                         "profiles/<kernel>_<workload>_counters.md")
    ap.add_argument("--summarize-parity", nargs=2, metavar=("JSONL", "COMMAND"),
                    help="no GPU work: turn the FA_PARITY_RECORD file of a GPU test run into "
                         "profiles/parity_gpu.md (+ .jsonl), recording COMMAND as its origin")
    ap.add_argument("--tile-order", type=int, default=0, choices=(0, 1, 2),
                    help="fused path only: workgroup-to-tile order of fa_fwd_tile_order (0 = fa_fwd's)")
    ap.add_argument("--eager", action="store_true",
                    help="time each launch between its own pair of events instead of one replay of the K "
                         "launches captured in a HIP graph (fused forward, --backward, --decode)")
    ap.add_argument("--all", action="store_true",
                    help="one JSON line per named forward workload (the benchmark line is the default run's)")
    ap.add_argument("--br", type=int, default=0, choices=(0, 128, 256),
                    help="fused path only: query rows per workgroup (fa_fwd_blocks); 0 = the selector's choice")
    ap.add_argument("--shape", metavar="B,H,N,d",
                    help="a shape outside the named workloads (seed 0, unit Gaussian inputs): B,H,N,d for the "
                         "forward or the backward, B,H,Nq,Nk,d with --decode")
    ap.add_argument("--summarize-io-sweep", metavar="DIR",
                    help="no GPU work: turn the FETCH_SIZE/WRITE_SIZE runs of the tile-order sweep under DIR "
                         "into profiles/fa_fwd_io_sweep.md (with --copy-calibration BYTES)")
    ap.add_argument("--backward", action="store_true",
                    help="the attention backward (dQ, dK, dV) on a prefill workload instead of the forward")
    ap.add_argument("--decode", action="store_true",
                    help="the decode-shaped forward (few queries against many keys) instead of the prefill "
                         "benchmark; also selects the decode kernels for --summarize-pmc")
    ap.add_argument("--gemm", action="store_true",
                    help="context, not the product: time a bf16 torch.mm (hipBLASLt) of M,N,K (--shape, default "
                         "8192,8192,8192, the forward benchmark's FLOP count) the same way")
    ap.add_argument("--memory", metavar="OUT_MD",
                    help="instead of timing: peak device memory of the fused and unfused forward over "
                         "a range of sequence lengths, written as a table to OUT_MD")
    args = ap.parse_args()
    if args.eager and (args.unfused or args.memory):
        ap.error("--eager applies to the fused forward, --backward and --decode")

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload, args.copy_calibration,
                      unfused=args.unfused, decode=args.decode, backward=args.backward)
        return
    if args.summarize_io_sweep:
        summarize_io_sweep(args.summarize_io_sweep, args.copy_calibration)
        return
    if args.summarize_parity:
        summarize_parity(*args.summarize_parity)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace[0], args.summarize_trace[1], args.workload, args.steps,
                        args.summarize_trace[2] if len(args.summarize_trace) > 2 else None)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.workload)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the forward shards over heads with no exchange between GPUs).", file=sys.stderr)
        sys.exit(2)

    if args.memory:
        memory_comparison(args.memory, "python3 bench.py --memory " + args.memory)
        return

    threads = str(len(os.sched_getaffinity(0)))
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ.setdefault(var, threads)

    if args.gemm:
        gemm_bench(args)
        return
    if args.decode:
        decode_bench(args)
        return
    if args.backward:
        backward_bench(args)
        return
    if args.all:
        import attn_inputs

        args.no_cpu_baseline = True
        for w in attn_inputs.WORKLOADS:
            args.workload = w.name
            fused_bench(args)
        return
    fused_bench(args)


def fused_bench(args):
    """Time the fused forward (or, with --unfused, the three-kernel baseline) on one
    workload and print its JSON line."""
    import torch

    import attn_inputs
    import io_aware_softmax_attn_amd as fa

    if args.shape:
        B, H, N, d = (int(x) for x in args.shape.split(","))
        w = attn_inputs.Workload(f"b{B}h{H}_n{N}_d{d}", B, H, N, d, seed=0)
    else:
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

    if args.copy_calibration:
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def launch(s=stream):
        if args.unfused:
            fa.fa_unfused_fwd(qg, kg, vg, o, lse, ws, scale=w.scale, stream=s)
        elif args.tile_order:
            fa.fa_fwd_tile_order(qg, kg, vg, o, lse, args.tile_order, scale=w.scale, stream=s)
        elif args.br:
            fa.fa_fwd_blocks(qg, kg, vg, o, lse, args.br, scale=w.scale, stream=s)
        else:
            fa.fa_fwd(qg, kg, vg, o, lse, scale=w.scale, stream=s)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()

    # The library allocates and clears nothing, so every launch records into the graph
    # as plain kernel nodes. The unfused baseline and the counter runs
    # (--launches-only) launch eagerly.
    use_graph = not (args.eager or args.unfused or args.launches_only)
    per_launch_ms, wall = time_launches(torch, launch, args.steps, stream, use_graph)
    avg_ms = sum(per_launch_ms) / len(per_launch_ms)
    step_ms = max(wall * 1e3 / args.steps, avg_ms)

    tflops = w.flops / (avg_ms * 1e-3) / 1e12
    traffic = None if (args.unfused or args.br or args.tile_order) else load_traffic(w.name)
    line = {
        "metric": metric_for(METRIC, f"B={w.B} H={w.H} N={w.N} d={w.d}"),
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
                   "path": "unfused-3-kernel" if args.unfused else "fused",
                   **({} if args.unfused else {"br": args.br or fa.fa_select_blocks(w.d, w.N, w.B, w.H)[0]}),
                   **({"tile_order": args.tile_order} if args.tile_order else {}),
                   "launch": "graph" if use_graph else "eager",
                   # every launch reads the same Q, K, V, which stay in the 256 MB Infinity Cache
                   # when they fit it; the kernel is compute-bound, so this moves the rate little
                   "inputs": "resident in HBM; the same buffers every launch (cache-warm)"},
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "kernel_ms_avg": round(avg_ms, 4),
            **timing_stats(per_launch_ms, use_graph, args.steps),
            "flops_per_launch": w.flops,
            "min_hbm_bytes_per_launch": w.min_hbm_bytes,
            # HBM rate of the counted bytes over the average launch, against the 8 TB/s roofline
            "hbm_gb_per_s": None if traffic is None else round(traffic / (avg_ms * 1e-3) / 1e9, 1),
            "hbm_frac_of_peak": None if traffic is None else round(traffic / (avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        },
    }
    if not args.launches_only and not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, q, k, v)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
