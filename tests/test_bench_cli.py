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


def test_unique_rows_count_a_shared_prefix_once():
    # three sequences sharing blocks 7 and 9 (32 tokens), then private blocks
    tables = np.array([[7, 9, 1], [7, 9, 2], [7, 9, -1]])
    lens = np.array([40, 35, 20])
    assert bench.unique_rows(lens, tables, 16) == 32 + (40 - 32) + (35 - 32)
    b = bench.algorithmic_bytes(lens, 4, 2, 64, 2, 2, 16, tables=tables)
    assert b["kv"] == 2 * (40 + 35 + 20) * 2 * 64 * 2
    assert b["kv_unique"] == 2 * 43 * 2 * 64 * 2
    assert b["partition_kernel"] - b["partition_kernel_unique"] == b["kv"] - b["kv_unique"]
    # without sharing the two agree
    t2 = np.array([[0, 1, 2], [3, 4, 5], [6, 7, -1]])
    b2 = bench.algorithmic_bytes(lens, 4, 2, 64, 2, 2, 16, tables=t2)
    assert b2["kv_unique"] == b2["kv"]


class _HostCase:
    """What cpu_baseline reads from a device case, held on the host: the tiny 4-sequence
    workload, with the 'GPU' output replaced by the oracle's own answer rounded to fp16."""

    def __init__(self):
        import torch

        import oracle
        from workloads import config_by_name, make_case
        self.cfg = cfg = config_by_name(1)
        self.case = case = make_case(cfg)
        kp, vp = case.k_pool.copy(), case.v_pool.copy()
        oracle.scatter(kp, vp, case.new_key, case.new_value, case.slot_mapping, 16)
        self.kp, self.vp = kp, vp
        ref = oracle.paged_decode(case.query, kp, vp, case.block_tables, case.lengths, cfg.scale, 16, "f16")
        self.out = torch.from_numpy(ref.astype(np.float16))

    def blocks_of(self, b):
        L = int(self.case.lengths[b])
        ids = self.case.block_tables[b, :max(1, -(-L // 16))]
        return self.kp[ids], self.vp[ids], np.arange(len(ids))


def test_cpu_baseline_runs_the_oracle_on_worker_processes():
    r = bench.cpu_baseline(_HostCase(), budget_s=0.3)
    assert r["kind"] == "oracle" and r["unit"] == "seqs/s" and r["value"] > 0
    assert 1 <= r["cores"] <= bench.MAX_ORACLE_WORKERS
    assert r["host"]["os_cpu_count"] == os.cpu_count()
    assert r["host"]["nproc"] == len(os.sched_getaffinity(0))
    assert "4 of 4 sequences" in r["sample"]
    assert r["max_abs_err_vs_gpu"] <= 2 ** -11 * 4      # fp16 rounding of |o| < 4
