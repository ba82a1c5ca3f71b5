"""The decode step captured in a HIP graph (torch.cuda.graph): the launches the benchmark
times -- the partition kernel with the new tokens written in, then the reduce, or the
shared-prefix step's kernels -- enqueue no memset and no host synchronisation, so
they capture; every replay, with the program's own eager work and synchronisations
between replays, gives the eager bits."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import paged_kv_cache_68_amd as pk  # noqa: E402
from workloads import config_by_name, make_case  # noqa: E402

from .gpu_helpers import DeviceCase, to_host_bits  # noqa: E402


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.mark.parametrize("cfg_idx", [2, 3])
def test_decode_step_in_a_graph(cfg_idx):
    cfg = config_by_name(cfg_idx)
    _say(f"graph capture: {cfg.name}")
    case = make_case(cfg, where="host" if cfg_idx == 2 else "device", poison=False)
    dc = DeviceCase(case)
    eager = to_host_bits(dc.step_append()).copy()
    pool_after = to_host_bits(dc.pool.k_cache(0)[:64]).copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm-up on the capture stream
        dc.step_append()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dc.step_append()
    scratch = torch.empty(1 << 20, device="cuda")
    for rep in range(4):
        dc.out.fill_(7.0)
        scratch.normal_()                          # the program's own work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(dc.out), eager), f"replay {rep}"
        assert np.array_equal(to_host_bits(dc.pool.k_cache(0)[:64]), pool_after)
    _say(f"  {cfg.name}: 4 replays equal the eager step")


@pytest.mark.parametrize("fuse", ["1", "0"], ids=["fused", "reduce"])
def test_shared_prefix_step_in_a_graph(monkeypatch, fuse):
    """The 64-fork step through paged_attention_decode_shared_prefix (prefix pass, then the
    suffix partitions with the cache write, which combine and write the output themselves,
    or whose partial results the cascade reduce combines): no memset, no host
    synchronisation; every replay gives the eager bits."""
    monkeypatch.setenv("PAGEDKV_CASCADE_FUSE", fuse)
    cfg = config_by_name(4)
    _say(f"graph capture, shared prefix: {cfg.name}")
    case = make_case(cfg, poison=False)
    dc = DeviceCase(case)
    P = pk.shared_prefix_blocks(case.block_tables, case.lengths, cfg.block_size, appending=True)
    step = pk.DecodeStep(dc.pool, 0, dc.out, dc.query, dc.tables, dc.lens, dc.new_key,
                         dc.new_value, scale=cfg.scale, partition_size=cfg.partition_size,
                         prefix_blocks=P)
    eager = to_host_bits(step()).copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    scratch = torch.empty(1 << 20, device="cuda")
    for rep in range(4):
        dc.out.fill_(7.0)
        scratch.normal_()                          # the program's own work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(dc.out), eager), f"replay {rep}"
    _say(f"  {cfg.name}: 4 replays equal the eager step")
