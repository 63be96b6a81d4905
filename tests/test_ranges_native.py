"""The decode kernel's range arithmetic (attn::Ranges in csrc/decode.hpp),
compiled for the host and checked against plain integer arithmetic: range
starts floor(i T / P) and the range holding each block, for block totals up
to 2^40 and range counts up to 4096 (tests/native/ranges_check.cpp).  No
GPU is needed."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                    reason="hipcc not available")
def test_ranges_arithmetic_is_exact(tmp_path):
    exe = tmp_path / "ranges_check"
    cmd = [HIPCC, "-O2", "-std=c++17", "--offload-host-only", "-x", "hip",
           "-I", os.path.join(ROOT, "causal_attention_amd", "csrc"),
           os.path.join(ROOT, "tests", "native", "ranges_check.cpp"),
           "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True,
                         timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout
