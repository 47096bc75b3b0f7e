"""bench.py command-line contract checks that need no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a configuration the library does not run


def test_summarize_trace_needs_no_gpu(tmp_path):
    """--summarize-trace turns a rocprofv3 stats CSV into a markdown summary that
    records the command; a minimal CSV is enough and no GPU is touched."""
    csv = tmp_path / "stats.csv"
    csv.write_text('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
                   '"unf_qk_kernel<128>",2,200000,100000.0,100.0,90000,110000,10000.0\n')
    (tmp_path / "profiles").mkdir()
    r = subprocess.run([sys.executable, "-c",
                        "import sys, bench; bench.ROOT = sys.argv[1]; "
                        "bench.summarize_trace(sys.argv[2], 'rocprofv3 ... -- python3 bench.py --unfused', None)",
                        str(tmp_path), str(csv)], capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    out = (tmp_path / "profiles" / "fa_unfused_b1h32_n8192_d128_kernel_trace.md").read_text()
    assert "`unf_qk_kernel<128>` | 2 | 100.0 |" in out
    assert "python3 bench.py --unfused" in out


def test_summarize_trace_reports_the_timed_launches(tmp_path):
    """With the per-dispatch trace next to the stats CSV, the fused summary also
    gives the average duration of the last `steps` launches and the gaps between
    them; the earlier (warmup) launches do not enter it."""
    name = "_ZN2fa12_GLOBAL__N_113fa_fwd_kernelILi128ELi2EEEvPKDF16b"
    (tmp_path / "fa_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        f'"{name}",5,5000000,1000000.0,100.0,800000,1400000,1.0\n')
    rows = ['"Kernel_Name","Start_Timestamp","End_Timestamp"']
    t = 0
    for dur, gap in ((1400000, 0), (1000000, 0), (800000, 10000), (800000, 20000), (1000000, 0)):
        rows.append(f'"{name}",{t},{t + dur}')
        t += dur + gap
    (tmp_path / "fa_kernel_trace.csv").write_text("\n".join(rows) + "\n")
    (tmp_path / "profiles").mkdir()
    r = subprocess.run([sys.executable, "-c",
                        "import sys, bench; bench.ROOT = sys.argv[1]; "
                        "bench.summarize_trace(sys.argv[2], 'rocprofv3 ... -- python3 bench.py', None, 3)",
                        str(tmp_path), str(tmp_path / "fa_kernel_stats.csv")],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    out = (tmp_path / "profiles" / "fa_fwd_b1h32_n8192_d128_kernel_trace.md").read_text()
    # last three: 800, 800, 1000 us -> 866.7 us; gaps between them 10 and 20 us -> 15 us
    assert "The last 3 launches (the timed region): 866.7 us per kernel on average (min 800.0, max 1000.0), " \
           "15.00 us between kernels" in out


def test_metric_names_the_shape_it_measures():
    """The default lines carry the metric names as quoted (their shapes are the
    benchmark shapes); other workloads carry their own shape in the name."""
    sys.path.insert(0, ROOT)
    import bench
    assert bench.metric_for(bench.METRIC, "B=1 H=32 N=8192 d=128") == bench.METRIC
    assert bench.metric_for(bench.BWD_METRIC, "B=1 H=32 N=8192 d=128") == bench.BWD_METRIC
    assert bench.metric_for(bench.DECODE_METRIC, "B=16 H=32 Nq=1 Nk=8192 d=128") == bench.DECODE_METRIC
    assert bench.metric_for(bench.METRIC, "B=4 H=16 N=1024 d=64").endswith(", B=4 H=16 N=1024 d=64")


def _committed_traffic():
    """(stem, workload, record) of every committed counter summary."""
    import glob
    import json

    out = []
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json"))):
        base = os.path.basename(path)[: -len("_traffic.json")]
        stem = "_".join(base.split("_")[:2])  # fa_fwd, fa_bwd, fa_decode, fa_unfused
        with open(path) as f:
            out.append((stem, base[len(stem) + 1:], json.load(f)))
    return out


def test_traffic_is_read_only_while_the_kernel_source_is_unchanged(tmp_path):
    """The bench line's HBM bytes come from a committed counter summary only while
    the hash recorded there matches the kernel source it was measured on; an edited
    source (here a copy with one byte appended) or a missing summary gives null."""
    sys.path.insert(0, ROOT)
    import bench

    srcs = {"fa_fwd": bench.KERNEL_SRC, "fa_bwd": bench.BWD_SRC, "fa_decode": bench.DECODE_SRC,
            "fa_unfused": bench.UNFUSED_SRC}
    recs = _committed_traffic()
    assert {stem for stem, _, _ in recs} >= {"fa_fwd", "fa_bwd", "fa_decode"}
    for stem, workload, rec in recs:
        src = srcs[stem]
        assert rec["workload"] == workload
        current = rec["kernel_source_sha256_16"] == bench.kernel_source_hash(src)
        got = bench.load_traffic(workload, stem, src)
        assert got == (rec["hbm_bytes_per_launch"] if current else None), (stem, workload)
        edited = tmp_path / os.path.basename(src)
        edited.write_bytes(open(src, "rb").read() + b"\n")
        assert bench.load_traffic(workload, stem, str(edited)) is None, (stem, workload)
    assert bench.load_traffic("no_such_workload", "fa_fwd") is None


def test_traffic_records_are_self_consistent():
    """Each summary's total is its fetch plus write bytes, and its ratio is that
    total over the read-once minimum it records."""
    for stem, workload, rec in _committed_traffic():
        assert rec["hbm_bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"] \
            or abs(rec["hbm_bytes_per_launch"] - rec["fetch_bytes_per_launch"] - rec["write_bytes_per_launch"]) <= 1
        ratio = rec["hbm_bytes_per_launch"] / rec["min_hbm_bytes_per_launch"]
        assert abs(ratio - rec["ratio_to_min"]) <= 1e-3 * ratio, (stem, workload)
        assert len(rec["commands"]) == 2 and "FETCH_SIZE" in rec["commands"][0] and "WRITE_SIZE" in rec["commands"][1]
