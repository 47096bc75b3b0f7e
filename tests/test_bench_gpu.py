"""bench.py's timing modes on a small shape (MI355X only).

The default timing captures the K launches in one HIP graph and replays it; --eager
issues them one by one. Both must print one well-formed JSON line, on the fused
forward, the backward and the decode-shaped forward."""
import json
import os
import subprocess
import sys

import pytest
import torch

from parity_util import announce

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*extra):
    announce("bench.py " + " ".join(extra))
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--no-cpu-baseline", *extra], capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("eager", [False, True])
def test_fused_line(eager):
    rec = run_bench("--shape", "1,4,1000,128", *(["--eager"] if eager else []))
    assert rec["config"]["launch"] == ("eager" if eager else "graph")
    assert rec["steps"] == 3 and rec["value"] > 0 and rec["roofline"]["kernel_ms_avg"] > 0
    r = rec["roofline"]
    # 3 steps: three graph replays of one launch, or three eager launches
    assert r["timing_samples"] == 3 and r["kernel_ms_min"] <= r["kernel_ms_median"] <= r["kernel_ms_max"]


@pytest.mark.parametrize("mode", ["--backward", "--decode"])
def test_backward_and_decode_lines(mode):
    rec = run_bench(mode, "--workload", "b1h1_n256_d64" if mode == "--backward" else "dec_b4h16_q4_k4096_d64")
    assert rec["config"]["launch"] == "graph" and rec["value"] > 0


def test_gemm_context_line():
    """The GEMM yardstick: one JSON line with the rate of a bf16 torch.mm of the given shape."""
    rec = run_bench("--gemm", "--shape", "512,256,1024")
    assert rec["config"] == {"op": "torch.mm", "M": 512, "N": 256, "K": 1024, "launch": "graph"}
    assert rec["value"] > 0 and rec["timing_samples"] == 3
    assert abs(rec["frac_of_peak"] - rec["value"] / 2516.6) < 1e-3
