"""The five decode-step workloads, as data.

Head shapes follow the models the pages use: Qwen2.5-0.5B (14 query heads, 2 KV
heads, head size 64) from "PagedAttention: Treating KV Memory Like Virtual Memory"
(the T4 measurements), Llama-3-8B (32/8/128) from "Why AI servers waste memory, and
how paging fixes it" ("How big it gets"), and Llama-2-70B (64/64/128, dense MHA)
from the footprint list in section 1 of "PagedAttention and Virtual Memory
Management". Block size 16 is the engine default all of them name.

Every length, table and value is drawn from ``numpy.random.default_rng(index)``
(and, for pools too large to build on the host, a seeded torch device generator),
so a case is fully determined by its config.
"""

from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class DecodeConfig:
    index: int            # 1-based; also the RNG seed
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str            # "f16" or "bf16": Q, new K / V and the output; K / V storage
                          # too unless kv_dtype is set
    block_size: int
    num_blocks: int       # physical blocks in the pool (one layer)
    batch: int
    lengths: str          # recipe name, see gen.draw_lengths
    partition_size: int   # tokens per split-context partition
    description: str
    kv_dtype: str = ""    # storage of K and V when it differs from ``dtype``: "fp8" (E4M3)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def kv(self) -> str:
        """Storage type of K and V ("f16", "bf16" or "fp8")."""
        return self.kv_dtype or self.dtype

    @property
    def elem_bytes(self) -> int:
        """Bytes per stored K / V element."""
        return 1 if self.kv == "fp8" else 2

    @property
    def scale(self) -> float:
        return 1.0 / float(self.head_dim) ** 0.5


CONFIGS = [
    DecodeConfig(
        index=1, name="tiny_qwen05b", num_q_heads=14, num_kv_heads=2, head_dim=64,
        dtype="f16", block_size=16, num_blocks=64, batch=4, lengths="fixed_1_16_17_40",
        partition_size=512,
        description="tiny single-layer decode, Qwen2.5-0.5B heads, lens {1,16,17,40}"),
    DecodeConfig(
        index=2, name="qwen05b_serving_b256", num_q_heads=14, num_kv_heads=2, head_dim=64,
        dtype="f16", block_size=16, num_blocks=58064, batch=256, lengths="lognormal_200",
        partition_size=512,
        description="Qwen2.5-0.5B serving batch of 256, lognormal lengths, 58,064-block pool"),
    DecodeConfig(
        index=3, name="llama3_8b_b64_ctx8192", num_q_heads=32, num_kv_heads=8, head_dim=128,
        dtype="bf16", block_size=16, num_blocks=40960, batch=64, lengths="const_8192",
        partition_size=512,
        description="Llama-3-8B heads (GQA 4), bf16, 64 sequences x 8,192 tokens"),
    DecodeConfig(
        index=4, name="llama3_8b_shared_prefix_b64", num_q_heads=32, num_kv_heads=8,
        head_dim=128, dtype="bf16", block_size=16, num_blocks=4096, batch=64,
        lengths="shared_prefix", partition_size=512,
        description="64 forks of a 4,103-token prefix (256 full shared blocks + CoW tail) "
                    "+ U[1,512] private tokens"),
    DecodeConfig(
        index=5, name="llama2_70b_mha_b512", num_q_heads=64, num_kv_heads=64, head_dim=128,
        dtype="f16", block_size=16, num_blocks=73728, batch=512, lengths="uniform_4096",
        partition_size=512,
        description="Llama-2-70B MHA heads, fp16, 512 sequences with U[1,4096] lengths"),
]


def config_by_name(name_or_index) -> DecodeConfig:
    for c in CONFIGS:
        if str(c.index) == str(name_or_index) or c.name == name_or_index \
                or f"c{c.index}" == str(name_or_index).lower():
            return c
    raise KeyError(name_or_index)
