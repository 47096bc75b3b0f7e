"""The C ABI's validation and dispatch layer (fa_api.cpp, fa_select.cpp), built for
the host with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and run
against stub launchers (tests/host/check_args_main.cpp). No GPU, no HIP."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "io_aware_softmax_attn_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_validation_layer_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "check_args")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", os.path.join(ROOT, "tests", "host", "check_args_main.cpp"),
           os.path.join(CSRC, "fa_api.cpp"), os.path.join(CSRC, "fa_select.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ)
    # A preloaded library ahead of the ASan runtime is tolerated; leaks are checked.
    env["ASAN_OPTIONS"] = "verify_asan_link_order=0:detect_leaks=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout[-4000:] + run.stderr[-4000:]
    assert "all passed" in run.stdout
