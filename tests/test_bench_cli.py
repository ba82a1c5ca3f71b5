"""bench.py's command line on the host: more than one GPU is refused with a message
before anything touches a device, and the algorithmic byte model adds up."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_of_the_headline_workload():
    # 64 sequences of 8,192 tokens, 32 query / 8 KV heads of 128, bf16, 16-token blocks
    lens = np.full(64, 8192)
    b = bench.algorithmic_bytes(lens, 32, 8, 128, 2, 2, 16)
    assert b["kv"] == 64 * 2 * 8192 * 8 * 128 * 2
    assert b["table"] == 64 * 4 * 512
    assert b["partition_kernel"] == 2148139264
    # the cache write of one token per sequence: K and V rows in and out, plus the slot
    assert b["write"] == 64 * (2 * 8 * 128 * 4 + 8)
    assert b["step"] == b["partition_kernel"] + b["o"] + b["write"]
