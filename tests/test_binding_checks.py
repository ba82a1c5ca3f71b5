"""The Python binding checks every tensor before calling the library (CPU only).

The C ABI receives addresses and counts but not buffer sizes, so a tensor of the wrong
type, shape, layout or device would let the kernels read or write outside it.  These
tests hand the binding such tensors and expect ValueError, with no call reaching the
library.  A stand-in pool object carries the geometry; the library is replaced by a
recorder, so nothing here needs a GPU.
"""

from types import SimpleNamespace

import pytest
import torch

import paged_kv_cache_68_amd as pk
from paged_kv_cache_68_amd import block_manager as pkbm

CPU = torch.device("cpu")


class _Recorder:
    """Stands in for the loaded library: records every call, returns KV_OK."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append(name)
            return 0
        return fn


@pytest.fixture
def rec(monkeypatch):
    r = _Recorder()
    monkeypatch.setattr(pk, "lib", lambda: r)
    monkeypatch.setattr(pkbm, "lib", lambda: r)
    monkeypatch.setattr(pk, "_stream", lambda s: 0)
    return r


def fake_pool(device=CPU, hkv=2, d=64, io=torch.float16, store=torch.float16, bs=16):
    """The attributes the binding reads from a KVPool."""
    return SimpleNamespace(handle=None, device=device,
                           device_index=-1 if device.type == "cpu" else device.index,
                           io_dtype=io, dtype=store, head_dim=d,
                           num_kv_heads=hkv, block_size=bs, desc=SimpleNamespace(block_size=bs),
                           memory=torch.empty(0, device="meta"))


def good_decode(B=3, hq=14, d=64, mb=4, io=torch.float16):
    return dict(out=torch.empty(B, hq, d, dtype=io), query=torch.zeros(B, hq, d, dtype=io),
                block_tables=torch.zeros(B, mb, dtype=torch.int32),
                context_lens=torch.ones(B, dtype=torch.int32))


def call_decode(pool, a, **kw):
    ws = kw.pop("workspace", torch.empty(16, dtype=torch.uint8))
    pk.paged_attention_partitions(pool, 0, a["out"], a["query"], a["block_tables"],
                                  a["context_lens"], workspace=ws, **kw)


def test_well_formed_call_reaches_the_library(rec):
    call_decode(fake_pool(), good_decode())
    assert rec.calls == ["paged_attention_partitions"]


@pytest.mark.parametrize("field,bad", [
    ("query", torch.zeros(3, 14, 128, dtype=torch.float16)),          # head size != pool's
    ("query", torch.zeros(3, 13, 64, dtype=torch.float16)),           # heads not a multiple of Hkv
    ("query", torch.zeros(3, 14, 64, dtype=torch.bfloat16)),          # not the pool's io dtype
    ("query", torch.zeros(3, 64, 14, dtype=torch.float16).transpose(1, 2)),   # strided
    ("out", torch.empty(3, 14, 32, dtype=torch.float16)),
    ("out", torch.empty(2, 14, 64, dtype=torch.float16)),
    ("out", torch.empty(3, 14, 64, dtype=torch.float32)),
    ("block_tables", torch.zeros(3, 4, dtype=torch.int64)),           # int64 tables
    ("block_tables", torch.zeros(3, 8, dtype=torch.int32)[:, ::2]),   # row stride != width
    ("block_tables", torch.zeros(2, 4, dtype=torch.int32)),           # fewer rows than the batch
    ("block_tables", torch.zeros(12, dtype=torch.int32)),             # 1-D
    ("context_lens", torch.ones(3, dtype=torch.int64)),
    ("context_lens", torch.ones(2, dtype=torch.int32)),
    ("query", [[0.0]]),                                               # not a tensor
])
def test_decode_rejects_bad_tensors(rec, field, bad):
    a = good_decode()
    a[field] = bad
    with pytest.raises(ValueError, match=field):
        call_decode(fake_pool(), a)
    assert rec.calls == []


def test_decode_rejects_tensors_off_the_pool_device(rec):
    with pytest.raises(ValueError, match="query"):
        call_decode(fake_pool(device=torch.device("cuda:0")), good_decode())
    assert rec.calls == []


def test_decode_rejects_a_strided_workspace(rec):
    with pytest.raises(ValueError, match="workspace"):
        call_decode(fake_pool(), good_decode(), workspace=torch.empty(64, dtype=torch.uint8)[::2])
    assert rec.calls == []


def test_scale_defaults_from_the_pool_head_size(rec, monkeypatch):
    seen = {}

    class Lib(_Recorder):
        def __getattr__(self, name):
            def fn(*args):
                seen["scale"] = args[9]
                return 0
            return fn
    monkeypatch.setattr(pk, "lib", lambda: Lib())
    call_decode(fake_pool(d=128), good_decode(d=128))
    assert seen["scale"] == pytest.approx(128 ** -0.5)


@pytest.mark.parametrize("which", ["new_key", "new_value"])
@pytest.mark.parametrize("bad", [torch.zeros(3, 2, 32, dtype=torch.float16),
                                 torch.zeros(2, 2, 64, dtype=torch.float16),
                                 torch.zeros(3, 2, 64, dtype=torch.bfloat16),
                                 None])
def test_append_rejects_bad_new_rows(rec, which, bad):
    a = good_decode()
    nk = {"new_key": torch.zeros(3, 2, 64, dtype=torch.float16),
          "new_value": torch.zeros(3, 2, 64, dtype=torch.float16)}
    nk[which] = bad
    with pytest.raises(ValueError):
        pk.paged_attention_partitions_append(fake_pool(), 0, a["out"], a["query"], nk["new_key"],
                                             nk["new_value"], a["block_tables"], a["context_lens"],
                                             workspace=torch.empty(16, dtype=torch.uint8))
    assert rec.calls == []


@pytest.mark.parametrize("field,bad", [
    ("slot_mapping", torch.zeros(4, dtype=torch.int32)),     # int32 slots (the kernel reads int64)
    ("slot_mapping", torch.zeros(4, 1, dtype=torch.int64)),
    ("key", torch.zeros(3, 2, 64, dtype=torch.float16)),     # fewer rows than slots
    ("key", torch.zeros(4, 2, 64, dtype=torch.bfloat16)),
    ("value", torch.zeros(4, 4, 64, dtype=torch.float16)),
    ("value", torch.zeros(4, 64, 2, dtype=torch.float16).transpose(1, 2)),
])
def test_reshape_and_cache_rejects_bad_tensors(rec, field, bad):
    a = {"key": torch.zeros(4, 2, 64, dtype=torch.float16),
         "value": torch.zeros(4, 2, 64, dtype=torch.float16),
         "slot_mapping": torch.zeros(4, dtype=torch.int64)}
    pk.reshape_and_cache(fake_pool(), 0, a["key"], a["value"], a["slot_mapping"])
    assert rec.calls == ["reshape_and_cache"]
    a[field] = bad
    with pytest.raises(ValueError, match=field):
        pk.reshape_and_cache(fake_pool(), 0, a["key"], a["value"], a["slot_mapping"])
    assert rec.calls == ["reshape_and_cache"]


def test_fp8_pool_takes_16_bit_rows(rec):
    pool = fake_pool(io=torch.bfloat16, store=torch.uint8)
    k = torch.zeros(2, 2, 64, dtype=torch.bfloat16)
    pk.reshape_and_cache(pool, 0, k, k.clone(), torch.zeros(2, dtype=torch.int64))
    with pytest.raises(ValueError, match="key"):
        pk.reshape_and_cache(pool, 0, k.to(torch.uint8), k, torch.zeros(2, dtype=torch.int64))
    assert rec.calls == ["reshape_and_cache"]


@pytest.mark.parametrize("field,bad", [
    ("query_start", torch.zeros(3, dtype=torch.int32)),      # batch + 1 entries expected
    ("query_start", torch.zeros(4, dtype=torch.int64)),
    ("context_lens", torch.ones(3, dtype=torch.int64)),
    ("block_tables", torch.zeros(2, 4, dtype=torch.int32)),
    ("out", torch.empty(9, 14, 64, dtype=torch.float16)),
    ("query", torch.zeros(10, 14, 128, dtype=torch.float16)),
])
def test_prefill_rejects_bad_tensors(rec, field, bad):
    a = {"out": torch.empty(10, 14, 64, dtype=torch.float16),
         "query": torch.zeros(10, 14, 64, dtype=torch.float16),
         "query_start": torch.tensor([0, 4, 8, 10], dtype=torch.int32),
         "block_tables": torch.zeros(3, 4, dtype=torch.int32),
         "context_lens": torch.ones(3, dtype=torch.int32)}
    pk.paged_attention_prefill(fake_pool(), 0, a["out"], a["query"], a["query_start"], 4,
                               a["block_tables"], a["context_lens"])
    assert rec.calls == ["paged_attention_prefill"]
    a[field] = bad
    with pytest.raises(ValueError, match=field):
        pk.paged_attention_prefill(fake_pool(), 0, a["out"], a["query"], a["query_start"], 4,
                                   a["block_tables"], a["context_lens"])
    assert rec.calls == ["paged_attention_prefill"]


def test_gather_output_must_hold_every_table_row(rec):
    t = torch.zeros(2, 3, dtype=torch.int32)
    ln = torch.ones(2, dtype=torch.int32)
    good = torch.empty(2, 48, 2, 64, dtype=torch.float16)
    pk.kv_pool_gather(fake_pool(), 0, t, ln, good, good.clone())
    with pytest.raises(ValueError, match="k_out"):
        pk.kv_pool_gather(fake_pool(), 0, t, ln, torch.empty(2, 47, 2, 64, dtype=torch.float16), good)
    assert rec.calls == ["kv_pool_gather"]


def test_copy_and_swap_pairs_are_checked(rec):
    pool = fake_pool()
    pk.copy_blocks(pool, torch.zeros(2, 3, dtype=torch.int32))
    for bad in (torch.zeros(2, 3, dtype=torch.int64), torch.zeros(2, 2, dtype=torch.int32),
                torch.zeros(3, 2, dtype=torch.int32).t()):
        with pytest.raises(ValueError, match="copies"):
            pk.copy_blocks(pool, bad)
    with pytest.raises(ValueError, match="pinned"):
        pk.swap_blocks(pool, pool, torch.zeros(2, 2, dtype=torch.int32))   # pageable host memory
    assert rec.calls == ["kv_copy_blocks"]


def test_host_pool_refuses_attention_calls(rec):
    pool = SimpleNamespace(host=True)
    with pytest.raises(ValueError, match="host memory"):
        pk.KVPool.device.fget(pool)


def test_decode_step_checks_once_and_calls_once(rec, monkeypatch):
    calls = []

    class Fn:
        def __init__(self, name):
            self.name = name

        def __call__(self, *args):
            calls.append((self.name, len(args)))
            return 0

    names = ["paged_attention_decode", "paged_attention_decode_append", "paged_attention_partitions",
             "paged_attention_partitions_append", "paged_attention_reduce"]
    monkeypatch.setattr(pk, "lib", lambda: SimpleNamespace(**{n: Fn(n) for n in names}))
    a = good_decode()
    ws = torch.empty(16, dtype=torch.uint8)
    step = pk.DecodeStep(fake_pool(), 0, a["out"], a["query"], a["block_tables"], a["context_lens"],
                         workspace=ws)
    step()
    step()
    nk = torch.zeros(3, 2, 64, dtype=torch.float16)
    s2 = pk.DecodeStep(fake_pool(), 0, a["out"], a["query"], a["block_tables"], a["context_lens"],
                       new_key=nk, new_value=nk.clone(), workspace=ws)
    s2()
    s2.partitions()
    s2.reduce()
    assert calls == [("paged_attention_decode", 14), ("paged_attention_decode", 14),
                     ("paged_attention_decode_append", 16), ("paged_attention_partitions_append", 16),
                     ("paged_attention_reduce", 14)]
    with pytest.raises(ValueError):
        pk.DecodeStep(fake_pool(), 0, a["out"], a["query"], a["block_tables"], a["context_lens"],
                      new_key=nk, workspace=ws)
    with pytest.raises(ValueError, match="block_tables"):
        pk.DecodeStep(fake_pool(), 0, a["out"], a["query"], a["block_tables"].long(),
                      a["context_lens"], workspace=ws)
