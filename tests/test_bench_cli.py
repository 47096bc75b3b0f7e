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
    assert r.stdout == ""  # no JSON line for a configuration this build does not run


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
