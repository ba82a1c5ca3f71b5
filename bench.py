#!/usr/bin/env python3
"""Benchmark one paged decode step on one MI355X and print one JSON line.

A step is the whole hot path over one batch: ``reshape_and_cache`` writes every
sequence's new token into its slot, then ``paged_attention_decode`` (partition kernel +
partition-reduce kernel) attends over the paged K/V, all on one stream.  Inputs are
seeded synthetic data built on the device before timing starts.

Default workload: Llama-3-8B heads (32 query / 8 KV, head 128, bf16), 64 sequences of
8,192 tokens, 16-token blocks scattered through a 40,960-block pool, partitions of 512.

Reported next to the whole-step rate:
* ``roofline``: algorithmic bytes of the partition kernel per launch divided by its
  average duration, timed with HIP events recorded on the stream it runs on;
* ``cpu_baseline``: the fp64 CPU oracle timed on a bounded sample of the same
  workload (it checks the kernel's output on those sequences too).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0                 # MI355X HBM3E, 8 TB/s
METRIC = "paged decode attention: seqs/s and achieved HBM GB/s (% of MI355X peak)"
PARTITION_KERNEL = "pa_partition"
PROFILE_DIR = os.path.join(ROOT, "profiles")


def unique_rows(lens, tables, block_size):
    """Distinct (physical block, slot) token rows a step reads: sequences that share
    blocks (forks of one prefix) read the shared rows once from HBM."""
    rows = []
    for b, L in enumerate(np.asarray(lens, dtype=np.int64).tolist()):
        t = np.arange(L, dtype=np.int64)
        rows.append(np.asarray(tables[b], dtype=np.int64)[t // block_size] * block_size + t % block_size)
    return int(np.unique(np.concatenate(rows)).size) if rows else 0


def algorithmic_bytes(lens, hq, hkv, d, kv_elem, io_elem=2, block_size=16, tables=None):
    """Bytes the method must move for one step (K+V of every context token, the table
    entries and length read, Q in and O out), and the partition kernel's share.
    kv_elem: bytes per stored K / V element (1 for FP8); io_elem: bytes per query /
    output / new key element.  With ``tables``, ``kv_unique`` counts each distinct
    token row once (the HBM bytes when sequences share blocks)."""
    lens = np.asarray(lens, dtype=np.int64)
    kv = int(np.sum(2 * lens * hkv * d * kv_elem))
    kv_unique = kv if tables is None else 2 * unique_rows(lens, tables, block_size) * hkv * d * kv_elem
    table = int(np.sum(4 * ((lens + block_size - 1) // block_size)))
    nlen = 4 * len(lens)
    q = len(lens) * hq * d * io_elem
    o = len(lens) * hq * d * io_elem
    write = len(lens) * (2 * hkv * d * (io_elem + kv_elem) + 8)
    return {"kv": kv, "kv_unique": kv_unique, "table": table, "lens": nlen, "q": q, "o": o,
            "partition_kernel": kv + table + nlen + q,
            "partition_kernel_unique": kv_unique + table + nlen + q,
            "write": write,
            "step": kv + table + nlen + q + o + write}


# the sources that decide the decode partition kernel's code and launch shape
DECODE_SOURCES = ("api.cpp", "device_common.h", "internal.h", "paged_decode.hip",
                  "paged_decode_mfma.hip", "partition_common.h")
# ... and those of the shared-prefix step (its prefix pass is the multi-token kernel)
CASCADE_SOURCES = DECODE_SOURCES + ("prefill_mfma.hip",)


def kernel_source_hash(names=DECODE_SOURCES) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_68_amd", "csrc")
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str = PARTITION_KERNEL):
    """HBM bytes per launch of the partition kernel (or per shared-prefix step, kernel
    "pa_cascade") from a committed rocprofv3 counter run
    (profiles/<kernel>_<workload>_traffic.json: TCC_EA0_RDREQ_DRAM_32B and
    TCC_EA0_WRREQ_WRITE_DRAM_32B, requests to DRAM counted in 32-byte units, so bytes =
    32 x count with no calibration), if taken on the current source."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    names = CASCADE_SOURCES if kernel == "pa_cascade" else DECODE_SOURCES
    if rec.get("kernel_source_hash") != kernel_source_hash(names):
        return None
    return rec.get("hbm_bytes_per_launch")


def host_cpu():
    """Host facts recorded with the CPU baseline."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"os_cpu_count": os.cpu_count(), "nproc": len(os.sched_getaffinity(0)), "model": model}


# Host cores the oracle may use: every one this process may run on, at most 16 (the
# host share of one GPU on the measuring machines).
MAX_ORACLE_WORKERS = 16


def _oracle_worker_init():
    from threadpoolctl import threadpool_limits
    global _BLAS_LIMIT
    _BLAS_LIMIT = threadpool_limits(limits=1)    # one BLAS thread per worker


def _oracle_task(task):
    """One sequence of the sample, read from the arrays the parent left in ``folder``."""
    import oracle
    folder, i, L, scale, B, kv, qdt = task
    kb = np.load(os.path.join(folder, f"k{i}.npy"), mmap_mode="r")
    vb = np.load(os.path.join(folder, f"v{i}.npy"), mmap_mode="r")
    q = np.load(os.path.join(folder, f"q{i}.npy"))
    table = np.arange(kb.shape[0])
    return i, oracle.paged_decode_seq(q, kb, vb, table, L, scale, B, kv, q_dtype=qdt)


def oracle_pool():
    """Worker processes for the CPU baseline, one per host core (at most 16), each with
    one BLAS thread.  Started as fresh interpreters before this process touches the GPU,
    so no worker ever holds GPU state."""
    import multiprocessing as mp
    workers = min(MAX_ORACLE_WORKERS, len(os.sched_getaffinity(0)))
    return mp.get_context("spawn").Pool(workers, initializer=_oracle_worker_init)


def cpu_baseline(dc, budget_s: float, pool=None, max_sample_bytes: int = 2 << 30):
    """Time the fp64 oracle on the host's cores (``pool``: worker processes from
    oracle_pool(), one BLAS thread each) on a bounded sample of the step: sequences
    taken at an even stride until their K/V reach ``max_sample_bytes``, the sample
    repeated until it is about ``budget_s`` seconds of CPU work.  Also checks the GPU
    output on the sample."""
    import shutil
    import tempfile

    import oracle
    from tests.device_case import to_host_bits   # plumbing: device bytes -> host bits

    cfg = dc.cfg
    lens = np.asarray(dc.case.lengths, dtype=np.int64)
    row = cfg.num_kv_heads * cfg.head_dim * cfg.elem_bytes * 2
    per_seq = np.maximum(lens, 1) * row
    n_fit = int(np.searchsorted(np.cumsum(np.sort(per_seq)), max_sample_bytes, side="right"))
    stride = max(1, -(-cfg.batch // max(1, n_fit)))
    sample = list(range(0, cfg.batch, stride))
    while len(sample) > 1 and int(per_seq[sample].sum()) > max_sample_bytes:
        sample = sample[:-1]
    out_bits = to_host_bits(dc.out)
    folder = tempfile.mkdtemp(prefix="pkv_oracle_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    try:
        for i in sample:
            kb, vb, _ = dc.blocks_of(i)
            np.save(os.path.join(folder, f"k{i}.npy"), kb)
            np.save(os.path.join(folder, f"v{i}.npy"), vb)
            np.save(os.path.join(folder, f"q{i}.npy"), dc.case.query[i])
        tasks = [(folder, i, int(lens[i]), cfg.scale, cfg.block_size, cfg.kv, cfg.dtype) for i in sample]
        own = pool is None
        if own:
            pool = oracle_pool()
        try:
            workers = pool._processes
            # an untimed pass over the sample gives its CPU cost, hence the passes timed
            t0 = time.perf_counter()
            results = pool.map(_oracle_task, tasks, chunksize=1)
            pass_cpu = (time.perf_counter() - t0) * min(workers, len(tasks))
            repeats = max(1, int(round(budget_s / max(pass_cpu, 1e-3))))
            t0 = time.perf_counter()
            pool.map(_oracle_task, tasks * repeats, chunksize=1)
            wall = time.perf_counter() - t0
        finally:
            if own:
                pool.close()
                pool.join()
    finally:
        shutil.rmtree(folder, ignore_errors=True)
    max_err = 0.0
    for i, ref in results:
        max_err = max(max_err, float(np.max(np.abs(oracle.to_f64(out_bits[i], cfg.dtype) - ref))))
    return {
        "value": len(tasks) * repeats / wall,
        "unit": "seqs/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{len(tasks)} of {cfg.batch} sequences of one step (every {stride}th), "
                  f"{repeats} pass(es), fp64 gather + softmax(qK^T)V, {workers} worker processes "
                  f"with one BLAS thread each, {wall:.1f} s wall",
        "host": host_cpu(),
        "max_abs_err_vs_gpu": max_err,
    }


# Copy-on-write block copies (kv_copy_blocks), Llama-3-8B pool geometry over all 32
# layers (8 KV heads x 128, bf16; 32 KiB per block per layer for K and for V).
COW_WORKLOADS = {
    # the first decode step after a 64-way fork of a 4,103-token prompt (the
    # shared-prefix workload): 63 streams copy the 7 rows of the shared tail block
    "llama3_8b_fork64_first_step": {"layers": 32, "blocks": 4096, "prompt": 4103, "forks": 64},
    # a beam-search style reshuffle: 1,024 whole-block copies
    "llama3_8b_cow_1024_blocks": {"layers": 32, "blocks": 4096, "copies": 1024, "rows": 16},
}


def bench_cow(args, name):
    import torch
    import paged_kv_cache_68_amd as pk

    w = COW_WORKLOADS[name]
    hkv, d, elem = 8, 128, 2
    row_bytes = hkv * d * elem
    pool = pk.KVPool(w["layers"], w["blocks"], hkv, d, "bf16")
    pool.memory.view(torch.int16).random_(-30000, 30000)
    if "prompt" in w:
        mgr = pk.BlockManager(w["blocks"], 16)
        mgr.add_request(0)
        mgr.append_batch([0], [w["prompt"]])
        for c in range(1, w["forks"]):
            mgr.fork(0, c)
        _, copies = mgr.append_batch(list(range(w["forks"])))
        # host cost of the block manager for one decode step of these streams
        t0 = time.perf_counter()
        for _ in range(200):
            mgr.append_batch(list(range(w["forks"])))
        host_us = (time.perf_counter() - t0) / 200 * 1e6
    else:
        rng = np.random.default_rng(7)
        perm = rng.permutation(w["blocks"])
        n = w["copies"]
        copies = np.stack([perm[:n], perm[n:2 * n], np.full(n, w["rows"])], axis=1).astype(np.int32)
        host_us = None
    copies_d = torch.from_numpy(np.ascontiguousarray(copies)).cuda()
    nbytes = int(2 * np.sum(copies[:, 2]) * row_bytes * 2 * w["layers"])   # read + write, K and V
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        pk.copy_blocks(pool, copies_d, stream)
    torch.cuda.synchronize()
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev_a[i].record(stream)
        pk.copy_blocks(pool, copies_d, stream)
        ev_b[i].record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(ev_a, ev_b)]))
    achieved = nbytes / (k_ms * 1e-3) / 1e9
    result = {
        "metric": "copy-on-write block copies (kv_copy_blocks): HBM GB/s, bytes read + written",
        "value": achieved, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "copies": int(copies.shape[0]),
                   "rows_per_copy": int(copies[0, 2]), **w},
        "roofline": {"bound": "hbm", "kernel": "cow_copy", "achieved": achieved,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": None, "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": k_ms * 1e3},
        "host_block_manager_us_per_decode_step": host_us,
    }
    if not args.no_cpu_baseline:
        import oracle
        # the oracle's copy on host arrays of two layers' K and V, scaled to all layers
        host = np.zeros((w["blocks"], 16, hkv, d), dtype=np.uint16)
        trip = [tuple(int(x) for x in c) for c in copies.tolist()]
        sample_layers = 2
        t0 = time.perf_counter()
        for _ in range(2 * sample_layers):
            oracle.copy_blocks(host, trip)
        t_cpu = (time.perf_counter() - t0) * w["layers"] / sample_layers
        result["cpu_baseline"] = {"value": nbytes / t_cpu / 1e9, "unit": "GB/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": f"{sample_layers} of {w['layers']} layers (K and V), "
                                            "scaled to all layers"}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


# Swap workloads (kv_swap_blocks): preempting one request by copying its blocks to a pool
# in pinned host memory and back, Llama-3-8B pool geometry over all 32 layers (8 KV heads
# x 128, bf16: 32 KiB per block per layer for K and for V).  The victim's device blocks
# are scattered over the pool, as an allocation history leaves them; its host blocks are
# the front of a fresh host free list.
SWAP_WORKLOADS = {
    # one 8,192-token request: 512 blocks, 1 GiB each way
    "llama3_8b_swap_8192_tokens": {"layers": 32, "dev_blocks": 4096, "host_blocks": 1024,
                                   "tokens": 8192},
    # a 2,407-token request: 151 blocks, 302 MiB each way
    "llama3_8b_swap_2407_tokens": {"layers": 32, "dev_blocks": 4096, "host_blocks": 1024,
                                   "tokens": 2407},
}
PEAK_HOST_LINK_GBPS = 64.0     # PCIe 5.0 x16, one direction (MI355X host interface)
LLC_BYTES = 256 << 20          # MI355X Infinity Cache
GRAPH_STEPS = 10               # decode steps per HIP graph in bench.py --graph


def bench_swap(args, name):
    import torch
    import paged_kv_cache_68_amd as pk

    w = SWAP_WORKLOADS[name]
    hkv, d, B = 8, 128, 16
    dev = pk.KVPool(w["layers"], w["dev_blocks"], hkv, d, "bf16")
    host = pk.KVPool(w["layers"], w["host_blocks"], hkv, d, "bf16", host=True)
    dev.memory.view(torch.int16).random_(-30000, 30000)
    # the block managers' moves give the pairs: the victim's table is a scattered set
    dev_m, host_m = pk.BlockManager(w["dev_blocks"], B), pk.BlockManager(w["host_blocks"], B)
    rng = np.random.default_rng(5)
    filler = int(rng.integers(w["dev_blocks"] // 4, w["dev_blocks"] // 2))
    dev_m.add_request(1)
    dev_m.append_batch([1], [filler * B])
    dev_m.add_request(0)
    for _ in range(w["tokens"]):                      # interleaved growth scatters blocks
        dev_m.append_batch([0, 1])
    out_pairs = dev_m.move_to(host_m, [0])
    in_pairs = host_m.move_to(dev_m, [0])
    n = int(out_pairs.shape[0])
    block_bytes = B * hkv * d * 2
    nbytes = n * block_bytes * 2 * w["layers"]       # one way: each byte crosses the link once
    out_d = torch.from_numpy(np.ascontiguousarray(out_pairs)).cuda()
    in_d = torch.from_numpy(np.ascontiguousarray(in_pairs)).cuda()
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        pk.swap_blocks(dev, host, out_d, stream)
        pk.swap_blocks(host, dev, in_d, stream)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        pk.swap_blocks(dev, host, out_d, stream)
        ev[i][1].record(stream)
        pk.swap_blocks(host, dev, in_d, stream)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    out_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    in_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    out_gbps = nbytes / (out_ms * 1e-3) / 1e9
    in_gbps = nbytes / (in_ms * 1e-3) / 1e9
    # the runtime copy (hipMemcpyAsync through torch) of one contiguous stretch of the
    # same size, for context
    stretch_dev = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    stretch_host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    for _ in range(2):
        stretch_host.copy_(stretch_dev, non_blocking=True)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record(stream)
    stretch_host.copy_(stretch_dev, non_blocking=True)
    e[1].record(stream)
    stretch_dev.copy_(stretch_host, non_blocking=True)
    e[2].record(stream)
    torch.cuda.synchronize()
    dma = {"d2h_GBps": nbytes / (e[0].elapsed_time(e[1]) * 1e-3) / 1e9,
           "h2d_GBps": nbytes / (e[1].elapsed_time(e[2]) * 1e-3) / 1e9}
    del stretch_dev, stretch_host
    value = 2 * nbytes / ((out_ms + in_ms) * 1e-3) / 1e9
    result = {
        "metric": "swap out + in of one request's blocks (kv_swap_blocks): host-link GB/s, "
                  "bytes moved each way",
        "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "blocks": n, "bytes_each_way": nbytes, **w},
        "swap_out": {"GBps": out_gbps, "avg_launch_us": out_ms * 1e3},
        "swap_in": {"GBps": in_gbps, "avg_launch_us": in_ms * 1e3},
        "contiguous_memcpy_same_bytes": dma,
        "roofline": {"bound": "host-link", "kernel": "swap_copy", "achieved": value,
                     "peak": PEAK_HOST_LINK_GBPS, "unit": "GB/s",
                     "frac": value / PEAK_HOST_LINK_GBPS, "traffic": None,
                     "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": (out_ms + in_ms) / 2 * 1e3},
    }
    if not args.no_cpu_baseline:
        import oracle
        # the oracle's block copies between host arrays of two layers' K and V, scaled
        src = np.zeros((w["dev_blocks"], B, hkv, d), dtype=np.uint16)
        dst = np.zeros((w["host_blocks"], B, hkv, d), dtype=np.uint16)
        pr = [tuple(int(x) for x in p) for p in out_pairs.tolist()]
        sample_layers = 2
        t0 = time.perf_counter()
        for _ in range(2 * sample_layers):
            oracle.swap_blocks(src, dst, pr)
        t_cpu = (time.perf_counter() - t0) * w["layers"] / sample_layers
        result["cpu_baseline"] = {"value": nbytes / t_cpu / 1e9, "unit": "GB/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": f"swap-out copies of {sample_layers} of {w['layers']} "
                                            "layers (K and V) between host arrays, scaled to all "
                                            "layers"}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


# Multi-token (prefill) attention workloads: chunks of new tokens attending causally over
# their sequences' paged K/V (the keys and values of the chunk already in the pool).
PREFILL_WORKLOADS = {
    # one 2,407-token prompt (151 blocks) in one chunk, Qwen2.5-0.5B heads, fp16
    "qwen05b_prompt_2407": {"hq": 14, "hkv": 2, "d": 64, "dtype": "f16", "chunks": [(2407, 2407)]},
    # a chunked-prefill step of 8,192 tokens: 4 sequences each computing positions
    # 6,144 .. 8,191 of an 8,192-token prompt, Llama-3-8B heads, bf16
    "llama3_8b_chunked_prefill_4x2048_ctx8192": {"hq": 32, "hkv": 8, "d": 128, "dtype": "bf16",
                                                 "chunks": [(2048, 8192)] * 4},
}
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}     # MI355X dense matrix-core peak


# Prefix-cache workloads (host bookkeeping, the kv_pc_* calls): admitting requests whose
# prompts share a prefix, then decode steps that append one token to each.
PREFIX_WORKLOADS = {
    # 64 requests of a 4,103-token prompt whose first 4,096 tokens (256 blocks) are the
    # same, then 256 decode steps of the 64 (Llama-3-8B-sized pool of 16-token blocks)
    "shared_prompt_64x4103_256_steps": {"requests": 64, "shared": 4096, "private": 7,
                                        "steps": 256, "blocks": 40960, "block_size": 16},
}


def bench_prefix_cache(args, name):
    """Host-side: the library's prefix cache through its Python binding (each call's
    marshalling included), and the oracle's for context on a smaller share."""
    import paged_kv_cache_68_amd as pk

    w = PREFIX_WORKLOADS[name]
    B, R = w["block_size"], w["requests"]
    rng = np.random.default_rng(11)
    shared = rng.integers(0, 128000, w["shared"], dtype=np.int32)
    prompts = [np.concatenate([shared, rng.integers(0, 128000, w["private"], dtype=np.int32)])
               for _ in range(R)]
    steps_tokens = rng.integers(0, 128000, (w["steps"], R), dtype=np.int32)

    def run(cache_cls, requests, steps, export):
        pc = cache_cls(w["blocks"], B)
        t0 = time.perf_counter()
        found = []
        for r in range(requests):
            f = pc.add_request(r, prompts[r])
            found.append(f)
            pc.append(r, prompts[r][f:])
        t_admit = time.perf_counter() - t0
        t0 = time.perf_counter()
        rids = list(range(requests))
        for s in range(steps):
            pc.append_step(rids, steps_tokens[s])
            if export:
                pc.export(list(range(requests)), -(-(w["shared"] + w["private"] + steps) // B))
        t_steps = time.perf_counter() - t0
        return found, t_admit, t_steps

    found, t_admit, t_steps = run(pk.PrefixCache, R, w["steps"], True)
    assert found[0] == 0 and all(f == w["shared"] for f in found[1:]), found[:4]
    hashed = w["shared"] + w["private"] + R * w["private"]      # tokens that were hashed or checked
    result = {
        "metric": "prefix cache (kv_pc_*): host us per admitted request and per decode step of "
                  "the batch",
        "value": t_steps * 1e6 / w["steps"], "unit": "us per decode step (append_step of 64 + export)",
        "n_gpus": 0, "steps": w["steps"], "warmup": 0, "ms_per_step": t_steps * 1e3 / w["steps"],
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": name, **w},
        "admit_us_per_request": t_admit * 1e6 / R,
        "prompt_tokens_per_s_admitted": R * (w["shared"] + w["private"]) / t_admit,
        "found_tokens": {"first": found[0], "others": found[1]},
        "roofline": None,
        "note": "host bookkeeping off the GPU path; each call crosses the Python binding "
                f"(a few us of marshalling per call); {hashed} distinct prompt tokens",
    }
    if not args.no_cpu_baseline:
        import oracle.prefix_cache as opc
        sample_steps = 32
        _, o_admit, o_steps = run(opc.PrefixCache, R, sample_steps, False)
        result["cpu_baseline"] = {"value": o_steps * 1e6 / sample_steps,
                                  "unit": "us per decode step (append_step of 64, no export)",
                                  "admit_us_per_request": o_admit * 1e6 / R, "cores": 1,
                                  "kind": "oracle", "sample": f"{sample_steps} of {w['steps']} steps"}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


def bench_prefill(args, name):
    import torch
    import oracle
    import paged_kv_cache_68_amd as pk

    w = PREFILL_WORKLOADS[name]
    hq, hkv, d, dt = w["hq"], w["hkv"], w["d"], w["dtype"]
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dt]
    ns = [n for n, _ in w["chunks"]]
    lens = np.array([L for _, L in w["chunks"]], dtype=np.int32)
    qs = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    nblk = [-(-int(L) // 16) for L in lens]
    nb = sum(nblk) + 64
    rng = np.random.default_rng(11)
    perm = rng.permutation(nb).astype(np.int32)
    tables = np.full((len(lens), max(nblk)), -1, dtype=np.int32)
    pos = 0
    for b, m in enumerate(nblk):
        tables[b, :m] = perm[pos:pos + m]
        pos += m
    kv = args.kv_dtype or dt
    pool = pk.KVPool(1, nb, hkv, d, kv, io_dtype=dt if kv == "fp8" else None)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    for c in (pool.k_cache(0), pool.v_cache(0)):
        if kv == "fp8":   # E4M3 codes of magnitude 2^-4 .. 2, either sign
            mag = torch.randint(0x20, 0x41, c.shape, generator=gen, device="cuda", dtype=torch.int32)
            sign = torch.randint(0, 2, c.shape, generator=gen, device="cuda", dtype=torch.int32) << 7
            c.copy_((mag | sign).to(torch.uint8))
        else:
            c.copy_(torch.randn(c.shape, generator=gen, device="cuda", dtype=torch.float32).to(tdt))
    q = torch.randn((int(qs[-1]), hq, d), generator=gen, device="cuda", dtype=torch.float32).to(tdt)
    out = torch.empty_like(q)
    qs_d = torch.from_numpy(qs).cuda()
    tab_d = torch.from_numpy(tables).cuda()
    lens_d = torch.from_numpy(lens).cuda()
    maxq = max(ns)
    stream = torch.cuda.current_stream()
    scale = 1.0 / math.sqrt(d)
    # the split entry point: the planner splits each row tile's keys over several
    # work-groups when the launch would leave the GPU idle (then a merge kernel follows)
    ws = pk.alloc_prefill_workspace(pool, len(lens), hq, int(qs[-1]), maxq, tables.shape[1])
    splits_used = bool(ws is not None)
    # work-groups per row tile: the workspace holds (acc, m, l) per row and split
    splits = 1 if ws is None else int(ws.numel() // (int(qs[-1]) * hq * (4 * d + 8)))
    run = lambda: pk.paged_attention_prefill_split(pool, 0, out, q, qs_d, maxq, tab_d, lens_d, scale,
                                                   workspace=ws, stream=stream)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev_a[i].record(stream)
        run()
        ev_b[i].record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(ev_a, ev_b)]))
    flops = oracle.prefill_flops(ns, lens, hq, d)
    tflops = flops / (k_ms * 1e-3) / 1e12
    tokens = int(qs[-1])
    result = {
        "metric": "paged prefill attention: query tokens/s and achieved TFLOP/s (% of MI355X dense matrix-core peak)",
        "value": tokens / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dt if kv == dt else f"{kv} kv, {dt} q/out", "data": "synthetic",
        "config": {"workload": name if kv == dt else f"{name}_{kv}kv", "q_heads": hq, "kv_heads": hkv,
                   "head_dim": d, "block_size": 16,
                   "chunks": [list(c) for c in w["chunks"]], "query_tokens": tokens,
                   "key_range_splits": splits},
        "roofline": {"bound": "mfma",
                     "kernel": "pa_prefill_mfma + pa_prefill_merge (key range split)" if splits_used
                     else "pa_prefill_mfma", "achieved": tflops,
                     "peak": PEAK_MFMA_TFLOPS[dt], "unit": "TFLOP/s", "frac": tflops / PEAK_MFMA_TFLOPS[dt],
                     "traffic": None, "algorithmic_flops_per_launch": flops, "avg_launch_us": k_ms * 1e3},
    }
    if not args.no_cpu_baseline:
        # the oracle on the first 8 query rows of the first sequence (the shortest rows,
        # which average the fewest values) and its last 8 (the costliest ones)
        from tests.device_case import to_host_bits
        kb = to_host_bits(pool.k_cache(0))
        vb = to_host_bits(pool.v_cache(0))
        qb = to_host_bits(q)
        n0, L0 = w["chunks"][0]
        rows = 8
        got_all = to_host_bits(out)
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            ref_last = oracle.paged_prefill_seq(qb[n0 - rows:n0], kb, vb, tables[0], L0, scale, 16, kv, q_dtype=dt)
            t_cpu = time.perf_counter() - t0
            # the first rows: query i of the chunk sits at position L0 - n0 + i
            ref_first = np.stack([oracle.paged_prefill_seq(qb[i:i + 1], kb, vb, tables[0], L0 - n0 + i + 1,
                                                           scale, 16, kv, q_dtype=dt)[0] for i in range(rows)])
        err_last = float(np.max(np.abs(oracle.to_f64(got_all[n0 - rows:n0], dt) - ref_last)))
        err_first = float(np.max(np.abs(oracle.to_f64(got_all[:rows], dt) - ref_first)))
        result["cpu_baseline"] = {"value": rows / t_cpu, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                                  "sample": f"the last {rows} query rows of sequence 0 ({t_cpu:.1f} s); "
                                            f"its first {rows} rows checked too",
                                  "max_abs_err_vs_gpu": max(err_last, err_first),
                                  "max_abs_err_first_rows": err_first, "max_abs_err_last_rows": err_last}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 100 untimed steps: the step time settles after a few dozen (the host-side launch path
    # warms up; the kernel itself is steady from the first steps)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="c3", help="workload: c1..c5 or a config name")
    ap.add_argument("--block-size", type=int, default=None,
                    help="rebuild the workload with this block size (8, 16, 32, 64); the pool "
                         "keeps the same number of token slots")
    ap.add_argument("--kv-dtype", choices=["fp8"], default=None,
                    help="store keys and values as FP8 (E4M3) instead of the workload's type")
    ap.add_argument("--prefill", choices=sorted(PREFILL_WORKLOADS),
                    help="time multi-token (prefill) attention on this workload instead")
    ap.add_argument("--cow", choices=sorted(COW_WORKLOADS),
                    help="time the copy-on-write block copy on this workload instead")
    ap.add_argument("--prefix-cache", choices=sorted(PREFIX_WORKLOADS), default=None,
                    help="host prefix-cache workload instead of the decode step")
    ap.add_argument("--swap", choices=sorted(SWAP_WORKLOADS),
                    help="time swap-out and swap-in block copies on this workload instead")
    ap.add_argument("--graph", action="store_true",
                    help="also time the decode step replayed from a HIP graph")
    ap.add_argument("--separate-write", action="store_true",
                    help="launch reshape_and_cache on its own instead of folding the cache "
                         "write into the partition kernel")
    ap.add_argument("--longest-first", action="store_true",
                    help="build the decode batch longest sequence first (kv_decode_order)")
    ap.add_argument("--no-shared-prefix", action="store_true",
                    help="for a batch of forks of one prefix, time the plain decode instead of "
                         "paged_attention_decode_shared_prefix")
    ap.add_argument("--cold", action="store_true",
                    help="also time each step after evicting the last-level cache (done by "
                         "default when the step's working set fits in it)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle CPU work (summed over the worker processes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain copy of known size (the cache-write kernel copying "
                         "512 MiB to consecutive slots), the reference for scaling rocprofv3 "
                         "FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(each GPU would run its own share of sequences independently).", file=sys.stderr)
        return 2

    if args.prefix_cache:          # host bookkeeping only
        return bench_prefix_cache(args, args.prefix_cache)

    # the CPU baseline's worker processes start before anything here touches the GPU
    decode_run = not (args.copy_calibration or args.cow or args.swap or args.prefill)
    workers = oracle_pool() if decode_run and not args.no_cpu_baseline else None
    try:
        return _main_gpu(args, workers)
    finally:
        if workers is not None:
            workers.close()
            workers.join()


def _main_gpu(args, workers):
    import torch
    import paged_kv_cache_68_amd as pk
    from workloads import config_by_name, is_fork, make_case
    from tests.device_case import DeviceCase

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.copy_calibration:
        # reshape_and_cache as a plain row copy: 131,072 rows of 2 KiB, K and V, to
        # consecutive slots -> 512 MiB read and 512 MiB written per launch
        T = 131072
        pool = pk.KVPool(1, T // 16, 8, 128, "bf16")
        key = torch.ones((T, 8, 128), dtype=torch.bfloat16, device="cuda")
        value = torch.ones_like(key)
        slots = torch.arange(T, dtype=torch.int64, device="cuda")
        for _ in range(3):
            pk.reshape_and_cache(pool, 0, key, value, slots)
        torch.cuda.synchronize()
        nbytes = 2 * T * 8 * 128 * 2
        print(json.dumps({"copy_calibration": {"kernel": "rc_scatter", "launches": 3,
                                               "bytes_read_per_launch": nbytes,
                                               "bytes_written_per_launch": nbytes}}))
        return 0

    if args.cow:
        return bench_cow(args, args.cow)
    if args.swap:
        return bench_swap(args, args.swap)
    if args.prefill:
        return bench_prefill(args, args.prefill)

    cfg = config_by_name(args.config)
    if args.block_size and args.block_size != cfg.block_size:
        import dataclasses
        B = args.block_size
        cfg = dataclasses.replace(cfg, block_size=B, num_blocks=cfg.num_blocks * cfg.block_size // B,
                                  name=f"{cfg.name}_b{B}")
    if args.kv_dtype:
        import dataclasses
        cfg = dataclasses.replace(cfg, kv_dtype=args.kv_dtype, name=f"{cfg.name}_{args.kv_dtype}kv")
    print(f"[bench] building {cfg.name} on the device", file=sys.stderr, flush=True)
    case = make_case(cfg, where="device" if cfg.index in (3, 5) else "host", poison=False)
    if args.longest_first:
        # the batch built in kv_decode_order's order (a scheduler's choice; the pools and
        # every sequence's data are unchanged)
        import dataclasses
        order = pk.decode_order(case.lengths)
        case = dataclasses.replace(case, lengths=case.lengths[order], block_tables=case.block_tables[order],
                                   slot_mapping=case.slot_mapping[order], query=case.query[order],
                                   new_key=case.new_key[order], new_value=case.new_value[order])
    dc = DeviceCase(case)
    nbytes = algorithmic_bytes(case.lengths, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                               cfg.elem_bytes, 2, cfg.block_size, tables=case.block_tables)
    stream = torch.cuda.current_stream()
    # Every workload writes each sequence's new token at position L - 1, so the cache write
    # can ride in the partition kernel (paged_attention_partitions_append); check that the
    # slot mapping is exactly that, else (or with --separate-write) launch it on its own.
    B = cfg.block_size
    table_slots = np.array([case.block_tables[b, (L - 1) // B] * B + (L - 1) % B if L > 0 else -1
                            for b, L in enumerate(case.lengths)], dtype=np.int64)
    fused = not args.separate_write and np.array_equal(table_slots, case.slot_mapping.astype(np.int64))
    if fused:
        # no slot index is read: the table entry the kernel reads anyway names the slot
        nbytes["write"] -= 8 * cfg.batch
        nbytes["step"] -= 8 * cfg.batch
        nbytes["partition_kernel"] += nbytes["write"]
        nbytes["partition_kernel_unique"] += nbytes["write"]

    # forks of one prefix: the shared-prefix entry point (the shared blocks read once for
    # the batch, as many as the tables share), unless --no-shared-prefix
    prefix_blocks = 0
    if is_fork(cfg) and not args.no_shared_prefix:
        prefix_blocks = pk.shared_prefix_blocks(case.block_tables, case.lengths, cfg.block_size,
                                                appending=fused)
    cascade = prefix_blocks > 0
    # the library combines in the suffix kernel when the table entries after the prefix
    # hold at most max(partition size, 1,024) tokens (else, or with PAGEDKV_CASCADE_FUSE=0,
    # a third kernel does)
    suffix_width = (case.block_tables.shape[1] - prefix_blocks) * cfg.block_size
    combined_in_suffix = (cascade and 0 < suffix_width <= max(cfg.partition_size, 1024)
                          and os.environ.get("PAGEDKV_CASCADE_FUSE", "1") != "0")

    # the step as a serving loop runs it: buffers checked once, one library call per step
    # (partitions, then the reduce when some sequence needs one)
    dstep = pk.DecodeStep(dc.pool, 0, dc.out, dc.query, dc.tables, dc.lens,
                          new_key=dc.new_key if fused else None,
                          new_value=dc.new_value if fused else None, scale=cfg.scale,
                          partition_size=cfg.partition_size,
                          workspace=None if cascade else dc.workspace, prefix_blocks=prefix_blocks)

    def step(on=None, ev_a=None, ev_b=None):
        st = stream if on is None else on
        if not fused:
            pk.reshape_and_cache(dc.pool, 0, dc.new_key, dc.new_value, dc.slots, st)
        if ev_a is None:
            dstep(st)
            return
        ev_a.record(st)
        if cascade:              # one call: the prefix pass and the suffixes (and the merge)
            dstep(st)
            ev_b.record(st)
            return
        dstep.partitions(st)
        ev_b.record(st)
        dstep.reduce(st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps); timing {args.steps}", file=sys.stderr, flush=True)

    # The K timed steps carry no events: on this stack a timing event is a marker the
    # command processor serialises (about 4.5 us of GPU time each), which would lengthen
    # short steps.  The partition kernel's own duration comes from K more steps with HIP
    # events recorded around it on its stream.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        step(ev_a=ev_a[i], ev_b=ev_b[i])
    torch.cuda.synchronize()
    part_times = [a.elapsed_time(b) for a, b in zip(ev_a, ev_b)]
    part_ms = float(np.median(part_times))
    # the kernel's HBM bytes: each distinct token row once (forks of a prefix share rows);
    # the shared-prefix step's kernels together also write the output once
    kernel_bytes = nbytes["partition_kernel_unique"] + (nbytes["o"] if cascade else 0)
    logical_bytes = nbytes["partition_kernel"] + (nbytes["o"] if cascade else 0)
    achieved = kernel_bytes / (part_ms * 1e-3) / 1e9
    effective = logical_bytes / (part_ms * 1e-3) / 1e9
    seqs_per_s = cfg.batch / (ms_step * 1e-3)
    print(f"[bench] {ms_step * 1e3:.1f} us/step, partition kernel {part_ms * 1e3:.1f} us "
          f"= {achieved:.0f} GB/s", file=sys.stderr, flush=True)

    traffic = load_traffic(cfg.name, "pa_cascade" if cascade else PARTITION_KERNEL)
    result = {
        "metric": METRIC,
        "value": seqs_per_s,
        "unit": "seqs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype if cfg.kv == cfg.dtype else f"{cfg.kv} kv, {cfg.dtype} q/out",
        "data": "synthetic",
        "config": {
            "workload": cfg.name,
            "batch": cfg.batch,
            "context_lens": "8192 each" if cfg.index == 3 else cfg.lengths,
            "q_heads": cfg.num_q_heads, "kv_heads": cfg.num_kv_heads, "head_dim": cfg.head_dim,
            "block_size": cfg.block_size, "pool_blocks": cfg.num_blocks,
            "partition_size": cfg.partition_size, "accumulate": "f32",
            "step": ("paged_attention_decode_shared_prefix (cache write folded in; "
                     f"{prefix_blocks} shared blocks)" if cascade else
                     "paged_attention_partitions_append (cache write folded in) + reduce" if fused
                     else "reshape_and_cache + paged_attention (partitions + reduce)"),
            "batch_order": "longest first (kv_decode_order)" if args.longest_first else "as generated",
        },
        "step_hbm_gbps": nbytes["step"] / (ms_step * 1e-3) / 1e9,
        "step_frac_of_peak": nbytes["step"] / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "roofline": {
            "bound": "hbm",
            "kernel": (("pa_prefill_mfma (dense prefix pass) + pa_partition_mfma (suffixes, "
                        "combined with the prefix and written), timed together")
                       if combined_in_suffix else
                       ("pa_prefill_mfma (dense prefix pass) + pa_partition_mfma (suffixes) + "
                        "pa_cascade_reduce, timed together") if cascade else PARTITION_KERNEL),
            "achieved": achieved,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kernel_bytes,
            "avg_launch_us": part_ms * 1e3,
            "launch_us_stat": f"median of {args.steps} HIP-event durations (mean "
                              f"{np.mean(part_times) * 1e3:.1f} us), events on the kernel's stream "
                              "in K steps run after the timed ones",
        },
    }
    if nbytes["partition_kernel"] != nbytes["partition_kernel_unique"]:
        # sequences share blocks: the roofline takes each distinct row once; the logical
        # rate (every sequence's rows, as if each were read from HBM) is reported beside it
        result["roofline"]["effective"] = {
            "achieved": effective, "unit": "GB/s",
            "logical_bytes_per_launch": logical_bytes,
            "note": "every sequence's K/V rows counted, shared rows once per sequence",
        }
    # --graph: also time the same step captured once in a HIP graph and replayed back to
    # back (how a serving loop might run short steps; each replay checked against the
    # eager output)
    if args.graph:
        # the step captured in HIP graphs and replayed back to back, one step per graph
        # and GRAPH_STEPS steps per graph: a graph launch costs a fixed amount of host and
        # command-processor time on this stack, which a longer graph spreads over its steps
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(on=side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        ref = dc.out.clone()
        result["graph_replay"] = {"how": "the step captured in a HIP graph (n steps per graph), "
                                         "graphs replayed back to back, every replay checked"}
        for n in (1, GRAPH_STEPS):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(n):
                    step(on=torch.cuda.current_stream())   # the capture stream
            for _ in range(args.warmup):
                graph.replay()
            torch.cuda.synchronize()
            dc.out.fill_(7.0)
            reps = max(1, args.steps // n)
            t0 = time.perf_counter()
            for _ in range(reps):
                graph.replay()
            torch.cuda.synchronize()
            g_ms = (time.perf_counter() - t0) * 1e3 / (reps * n)
            assert torch.equal(dc.out.view(torch.int16), ref.view(torch.int16)), "graph replay differs"
            result["graph_replay"][f"{n}_steps_per_graph"] = {
                "us_per_step": g_ms * 1e3, "seqs_per_s": cfg.batch / (g_ms * 1e-3)}
            del graph
    # A working set smaller than the 256 MB Infinity Cache is served from it when steps
    # run back to back.  For such workloads also time each step cold: a 512 MiB write
    # between steps evicts the cache, and HIP events bracket the step alone.
    tabs = dc.tables[dc.tables >= 0]
    footprint = int(torch.unique(tabs).numel()) * cfg.block_size * cfg.num_kv_heads * cfg.head_dim * cfg.elem_bytes * 2
    if footprint < LLC_BYTES or args.cold:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.steps):
            flush.fill_(i & 0xFF)
            ev[i][0].record(stream)
            step()
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        step_us = float(np.median([e[0].elapsed_time(e[2]) for e in ev])) * 1e3
        result["cold_cache"] = {
            "how": "512 MiB write between steps; median of HIP-event times of the step alone",
            "unique_kv_bytes": footprint,
            "us_per_step": step_us,
            "seqs_per_s": cfg.batch / (step_us * 1e-6),
            "step_hbm_gbps": nbytes["step"] / (step_us * 1e-6) / 1e9,
            "step_frac_of_peak": nbytes["step"] / (step_us * 1e-6) / 1e9 / PEAK_HBM_GBPS,
            "unique_kv_gbps": footprint / (step_us * 1e-6) / 1e9,
        }
        del flush
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(dc, args.cpu_budget, workers)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
