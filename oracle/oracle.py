"""Plain, slow, fp64 CPU definition of one paged decode step.

TEST INFRASTRUCTURE ONLY: called by tests/, by __graft_entry__.smoke() and by the
cpu_baseline leg of bench.py.  It shares no code with the HIP path and imports
nothing from it.

Sources (page title, then the section / equation / figure used):

[P1] "PagedAttention: Treating KV Memory Like Virtual Memory" — "How the kernel
     reads a block table" (the address equation; the per-tile cost of the Qwen
     shape: 64 B of block numbers, 4 KiB of K+V, 14,336 multiply-adds).
[P2] "Why AI servers waste memory, and how paging fixes it" — "How big it gets"
     (bytes per token), "The idea: a block table" (position p -> block p // B,
     slot p % B; Figure 3), "The real implementation" (append writes the token into
     slot `offset` of the last block), "Reading through the table" (two-pass
     reference attention), "Proof it works" (paged == contiguous).
[P3] "PagedAttention and Virtual Memory Management: Mathematical Foundations ..."
     — section 1 (M_KV closed form), section 3 (j = floor(t/B), o = t mod B, the
     t = 38 example, bytes per physical block), section 4 (Addr_K / Addr_V, the
     block-wise online-softmax decode, and the cross-block reduction formula),
     section 5 (the copy-on-write copy of the rows a shared block already holds).

Readings where the pages are silent or garbled:
* GQA: query head h reads KV head h // G with G = Hq / Hkv (contiguous groups).
  The einsum pair in P3 section 4 would mix every query head with every KV head;
  that is taken as a transcription slip.
* ``lengths`` include the token just written by the cache write.
* The output of a sequence with no tokens (L = 0) is defined as zeros.
* Stored values are fp16 / bf16 bit patterns; they are widened to fp64 exactly and
  every step below is done in fp64 without rounding back.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "to_f64", "fp8_to_f64", "encode_fp8", "quantize_fp8", "FP8_MAX", "kv_bytes_per_token",
    "kv_pool_bytes", "block_bytes", "locate",
    "physical_address", "scatter", "copy_blocks", "swap_blocks", "gather", "attention_contiguous", "softmax_weights",
    "paged_decode", "paged_decode_seq", "online_decode_seq", "partition_partials",
    "combine_partials", "partitioned_decode_seq", "brute_force_seq", "paged_prefill_seq",
    "paged_prefill", "prefill_flops",
]


# ---------------------------------------------------------------- storage types

def to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Stored bit patterns -> exact float64 values: uint16 of fp16 / bf16, or uint8
    codes of fp8 (E4M3, see ``fp8_to_f64``)."""
    if dtype == "fp8":
        return fp8_to_f64(bits)
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# FP8 keys and values (one byte per element: b = 1 in P3 section 1).  The pages fix only
# the width; the format taken is the 8-bit E4M3 layout with 1 sign bit, 4 exponent bits
# (bias 7) and 3 mantissa bits, no infinities, and S.1111.111 as NaN, so the largest
# finite magnitude is 1.75 * 2**8 = 448.  No scale factor is applied.

FP8_MAX = 448.0


def fp8_to_f64(codes: np.ndarray) -> np.ndarray:
    """uint8 E4M3 codes -> exact float64 values (exponent field 0: subnormal m * 2**-9)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def encode_fp8(x: np.ndarray) -> np.ndarray:
    """float64 values -> uint8 E4M3 codes: round to nearest, ties to the even code;
    magnitudes past 448 (and infinities) saturate to 448; NaN -> S.1111.111 with the
    input's sign.  Each value is rounded on the grid of its binade (the subnormal grid
    2**-9 below 2**-6); every scaling below is by a power of two, so exact in fp64, and
    ``np.rint`` rounds halves to even."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    a = np.abs(np.where(np.isnan(x), 0.0, x))
    # normal binades: a = m * 2**e with m in [1, 2); 3 mantissa bits
    _, E = np.frexp(np.where((a > 0) & np.isfinite(a), a, 1.0))
    e = E.astype(np.int64) - 1
    q = np.rint((np.ldexp(np.where(np.isfinite(a), a, 1.0), -e) - 1.0) * 8.0).astype(np.int64)
    e = np.where(q == 8, e + 1, e)
    q = np.where(q == 8, 0, q)
    normal = ((e + 7) << 3) | q
    # subnormal grid below 2**-6: code m = a / 2**-9 rounded (8 is the smallest normal)
    sub = np.rint(np.where(a < 2.0 ** -6, a, 0.0) / 2.0 ** -9).astype(np.int64)
    code = np.where(a < 2.0 ** -6, sub, np.minimum(normal, 0x7E))
    code = np.where(a >= FP8_MAX, 0x7E, code)                        # saturate, incl. inf
    code = np.where(np.isnan(x), 0x7F, code)
    return (code | sign).astype(np.uint8)


def quantize_fp8(bits: np.ndarray, src_dtype: str) -> np.ndarray:
    """16-bit key / value rows (fp16 or bf16 bit patterns) -> E4M3 codes, element-wise
    (the cache write of an FP8 pool)."""
    return encode_fp8(to_f64(bits, src_dtype))


# ---------------------------------------------------------------- footprint

def kv_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """M_KV(1) = 2 * N_L * N_KV * d_h * b   [P3 section 1; P2 "How big it gets"]."""
    return 2 * n_layers * n_kv_heads * head_dim * elem_bytes


def kv_pool_bytes(n_layers, n_kv_heads, head_dim, elem_bytes, num_blocks, block_size) -> int:
    """Bytes of a pool of ``num_blocks`` blocks of ``block_size`` token slots."""
    return kv_bytes_per_token(n_layers, n_kv_heads, head_dim, elem_bytes) * num_blocks * block_size


def block_bytes(n_kv_heads, head_dim, elem_bytes, block_size, n_layers=1) -> int:
    """Bytes of one physical block, K and V   [P3 section 3, "Physical Block Representation"]."""
    return 2 * n_layers * n_kv_heads * head_dim * block_size * elem_bytes


# ---------------------------------------------------------------- indexing

def locate(t: int, block_size: int, table) -> tuple[int, int, int]:
    """Token position t -> (logical block j, offset o, physical block T[j]).

    j = floor(t / B), o = t mod B   [P3 section 3; P2 "The idea: a block table"].
    """
    j = t // block_size
    o = t % block_size
    return j, o, int(table[j])


def physical_address(t, block_size, table, stride_block, stride_token, head=0, stride_head=0,
                     base=0):
    """Addr(t) = base + T[t // B] * stride_block + (t mod B) * stride_token + h * stride_head

    [P3 section 4, Addr_K / Addr_V; P1 "How the kernel reads a block table"].
    """
    j, o, p = locate(t, block_size, table)
    return base + p * stride_block + o * stride_token + head * stride_head


# ---------------------------------------------------------------- cache write

def scatter(k_pool: np.ndarray, v_pool: np.ndarray, key: np.ndarray, value: np.ndarray,
            slot_mapping: np.ndarray, block_size: int) -> None:
    """Write token i's K and V rows into slot ``slot_mapping[i]`` of the pools, in place.

    slot = physical block * B + offset; the row lands in block slot // B at offset
    slot mod B   [P2 "The real implementation": the append writes into slot `offset`
    of the last block; P3 section 5, case 1].  A pure copy of the stored bits.
    """
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        blk, off = int(slot) // block_size, int(slot) % block_size
        k_pool[blk, off] = key[i]
        v_pool[blk, off] = value[i]


def copy_blocks(pool: np.ndarray, copies) -> None:
    """Copy-on-write copies, in place: for each (src, dst, rows), the first ``rows``
    token rows of physical block src are copied into block dst; the other rows of dst
    are left as they were   [P3 section 5, case 2: copy the o token vectors already in
    p to p_new].  ``pool`` is one K or V cache, block index first.  A pure copy of the
    stored bits; pairs are applied in order.
    """
    for src, dst, rows in copies:
        pool[int(dst), :int(rows)] = pool[int(src), :int(rows)]


def swap_blocks(src_pool: np.ndarray, dst_pool: np.ndarray, pairs) -> None:
    """Swap copies between two pools of the same block shape (device and host), in
    place: for each (src, dst), every token row of block src of ``src_pool`` is copied
    into block dst of ``dst_pool``   [P3 section 6, swapping: the victim's physical
    blocks go to a block pool in host memory, and come back the same way].  ``src_pool``
    and ``dst_pool`` are one K or V cache each, block index first.  A pure copy of the
    stored bits, pairs applied in order.
    """
    for src, dst in pairs:
        dst_pool[int(dst)] = src_pool[int(src)]


def gather(pool: np.ndarray, table, length: int, block_size: int) -> np.ndarray:
    """Copy a sequence's first ``length`` token rows into a contiguous array.

    Row t comes from physical block T[t // B], slot t mod B   [P2 "Reading through
    the table"; P3 section 3].  Returns the stored values unchanged, shape
    [length, *pool.shape[2:]].
    """
    rows = []
    for t in range(int(length)):
        j, o, p = locate(t, block_size, table)
        rows.append(pool[p, o])
    if not rows:
        return np.zeros((0,) + pool.shape[2:], dtype=pool.dtype)
    return np.stack(rows)


# ---------------------------------------------------------------- attention

def softmax_weights(scores: np.ndarray) -> np.ndarray:
    """exp(s - max s) / sum exp(s - max s)  along the last axis, fp64."""
    m = scores.max(axis=-1, keepdims=True)
    e = np.exp(scores - m)
    return e / e.sum(axis=-1, keepdims=True)


def attention_contiguous(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """One sequence's decode attention on contiguous K/V, fp64.

    q: [Hq, d]; k, v: [L, Hkv, d].  Query head h uses KV head h // G.
    Scores s_t = scale * q_h . k_t, weights = softmax(s), o_h = sum_t w_t v_t
    [P2 "Reading through the table": scores, max-subtracted exponentials, normalised
    weights, weighted sum of values].
    """
    hq, d = q.shape
    L, hkv, _ = k.shape
    if L == 0:
        return np.zeros((hq, d), dtype=np.float64)
    g = hq // hkv
    out = np.empty((hq, d), dtype=np.float64)
    for h in range(hq):
        kv = h // g
        s = (k[:, kv, :] @ q[h]) * scale          # [L]
        w = softmax_weights(s)
        out[h] = w @ v[:, kv, :]
    return out


def paged_decode_seq(q_bits, k_pool_bits, v_pool_bits, table, length, scale, block_size, dtype,
                     q_dtype=None):
    """Decode one sequence: gather K/V through its table, then contiguous attention.
    ``dtype`` is the pools' storage type, ``q_dtype`` the query's (default: the same)."""
    kc = to_f64(gather(k_pool_bits, table, length, block_size), dtype)
    vc = to_f64(gather(v_pool_bits, table, length, block_size), dtype)
    return attention_contiguous(to_f64(q_bits, q_dtype or dtype), kc, vc, scale)


def paged_decode(query_bits, k_pool_bits, v_pool_bits, block_tables, lengths, scale,
                 block_size, dtype, seqs=None, q_dtype=None) -> np.ndarray:
    """Whole batch (or the sequences listed in ``seqs``): fp64 [n, Hq, d]."""
    idx = range(len(lengths)) if seqs is None else seqs
    return np.stack([
        paged_decode_seq(query_bits[b], k_pool_bits, v_pool_bits, block_tables[b],
                         int(lengths[b]), scale, block_size, dtype, q_dtype)
        for b in idx])


# ---------------------------------------------------------------- online / partitioned forms

def online_decode_seq(q, k_pool, v_pool, table, length, scale, block_size):
    """Block-by-block online softmax over the table, fp64   [P3 section 4 decode pass].

    q: [Hq, d] float64; pools float64 [nb, B, Hkv, d].  Running max m, running sum l
    and accumulator acc per query head; each block rescales the old state by
    exp(m_old - m_new) and adds its own exponentials.  Returns acc / l.
    """
    hq, d = q.shape
    hkv = k_pool.shape[2]
    g = hq // hkv
    heads_kv = np.arange(hq) // g
    m = np.full(hq, -np.inf)
    l = np.zeros(hq)
    acc = np.zeros((hq, d))
    n_blocks = -(-int(length) // block_size)
    for j in range(n_blocks):
        p = int(table[j])
        n = min(block_size, int(length) - j * block_size)
        kb = k_pool[p, :n][:, heads_kv, :]      # [n, Hq, d]: each q head's KV rows
        vb = v_pool[p, :n][:, heads_kv, :]
        s = np.einsum("hd,nhd->hn", q, kb) * scale
        m_new = np.maximum(m, s.max(axis=1))
        alpha = np.exp(m - m_new)
        e = np.exp(s - m_new[:, None])
        l = alpha * l + e.sum(axis=1)
        acc = alpha[:, None] * acc + np.einsum("hn,nhd->hd", e, vb)
        m = m_new
    if n_blocks == 0:
        return np.zeros((hq, d))
    return acc / l[:, None]


def partition_partials(q, k_pool, v_pool, table, length, scale, block_size, partition_size):
    """Per partition k of ``partition_size`` tokens: (m_k, l_k, acc_k), fp64.

    m_k = max score in the partition, l_k = sum exp(s - m_k), acc_k = sum exp(s - m_k) v
    (so the partition's own output is O_k = acc_k / l_k).
    """
    hq, d = q.shape
    hkv = k_pool.shape[2]
    g = hq // hkv
    out = []
    L = int(length)
    for start in range(0, L, partition_size):
        stop = min(L, start + partition_size)
        rows = [locate(t, block_size, table) for t in range(start, stop)]
        kk = np.stack([k_pool[p, o] for _, o, p in rows])    # [n, Hkv, d]
        vv = np.stack([v_pool[p, o] for _, o, p in rows])
        m_k = np.empty(hq)
        l_k = np.empty(hq)
        acc_k = np.empty((hq, d))
        for h in range(hq):
            s = (kk[:, h // g, :] @ q[h]) * scale
            m_k[h] = s.max()
            e = np.exp(s - m_k[h])
            l_k[h] = e.sum()
            acc_k[h] = e @ vv[:, h // g, :]
        out.append((m_k, l_k, acc_k))
    return out


def combine_partials(partials):
    """Cross-partition reduction   [P3 section 4, "Cross-Block Reduction Kernel"].

    m_g = max_k m_k, l_g = sum_k l_k exp(m_k - m_g),
    O = sum_k (l_k exp(m_k - m_g) / l_g) O_k  with O_k = acc_k / l_k.
    """
    ms = np.stack([p[0] for p in partials])           # [P, Hq]
    ls = np.stack([p[1] for p in partials])
    os_ = np.stack([p[2] / p[1][:, None] for p in partials])   # O_k, [P, Hq, d]
    m_g = ms.max(axis=0)
    w = ls * np.exp(ms - m_g)
    l_g = w.sum(axis=0)
    return np.einsum("ph,phd->hd", w / l_g, os_)


def partitioned_decode_seq(q, k_pool, v_pool, table, length, scale, block_size, partition_size):
    if int(length) == 0:
        return np.zeros_like(q)
    return combine_partials(partition_partials(q, k_pool, v_pool, table, length, scale,
                                               block_size, partition_size))


# ---------------------------------------------------------------- brute force (tiny inputs)

def brute_force_seq(q, keys, values, scale):
    """softmax(q K^T * scale) V with pure-Python loops and no max subtraction.

    q: list over query heads of length-d lists; keys/values: list over tokens of
    [Hkv][d] nested lists.  For tiny inputs only (|scores| small, so plain exp is safe).
    """
    hq = len(q)
    hkv = len(keys[0])
    g = hq // hkv
    d = len(q[0])
    out = []
    for h in range(hq):
        kv = h // g
        ex = []
        for t in range(len(keys)):
            dot = 0.0
            for i in range(d):
                dot += q[h][i] * keys[t][kv][i]
            ex.append(math.exp(dot * scale))
        z = math.fsum(ex)
        row = []
        for i in range(d):
            row.append(math.fsum(ex[t] * values[t][kv][i] for t in range(len(keys))) / z)
        out.append(row)
    return out


# ---------------------------------------------------------------- multi-token queries (prefill)

def paged_prefill_seq(q_bits, k_pool_bits, v_pool_bits, table, length, scale, block_size, dtype,
                      q_dtype=None):
    """The n = len(q_bits) newest tokens of one sequence attend over the sequence's paged
    K/V, causally: token i sits at position p = length - n + i and its query heads see
    positions [0, p] only.  Their own keys and values are already in the pool.

    A prompt (or a chunk of one) processed in parallel, as "PagedAttention: Treating KV
    Memory Like Virtual Memory", section "What the allocator actually sees" (a request
    also comes as a whole prompt, or as pieces of one cut to the step's token budget),
    and "PagedAttention and Virtual Memory Management" (prefill processes the prompt in
    parallel) describe it; each row is
    the attention of P2 "Reading through the table" over the first p + 1 positions.
    Tokens with p < 0 (more queries than the length holds) get zero output.
    q_bits: [n, Hq, d].  Returns fp64 [n, Hq, d].
    """
    n = len(q_bits)
    qf = to_f64(q_bits, q_dtype or dtype)
    kc = to_f64(gather(k_pool_bits, table, length, block_size), dtype)
    vc = to_f64(gather(v_pool_bits, table, length, block_size), dtype)
    out = np.zeros(qf.shape, dtype=np.float64)
    for i in range(n):
        p = int(length) - n + i
        if p >= 0:
            out[i] = attention_contiguous(qf[i], kc[:p + 1], vc[:p + 1], scale)
    return out


def paged_prefill(query_bits, query_start, k_pool_bits, v_pool_bits, block_tables, lengths, scale,
                  block_size, dtype, q_dtype=None, seqs=None) -> np.ndarray:
    """A batch of chunks: sequence b's queries are rows [query_start[b], query_start[b+1])
    of ``query_bits`` ([T, Hq, d]).  Returns fp64 [T, Hq, d] (rows of skipped sequences
    are zero)."""
    out = np.zeros(np.asarray(query_bits).shape, dtype=np.float64)
    idx = range(len(lengths)) if seqs is None else seqs
    for b in idx:
        a, e = int(query_start[b]), int(query_start[b + 1])
        if e > a:
            out[a:e] = paged_prefill_seq(query_bits[a:e], k_pool_bits, v_pool_bits, block_tables[b],
                                         int(lengths[b]), scale, block_size, dtype, q_dtype)
    return out


def prefill_flops(query_lens, lengths, num_q_heads, head_dim) -> int:
    """Multiply-adds x 2 of the causal attention above: a query at position p costs
    (p + 1) * d for q.K and as many for P.V, per query head."""
    total = 0
    for n, L in zip(query_lens, lengths):
        n, L = int(n), int(L)
        first = max(0, L - n)                   # position of the first query (clamped)
        # sum over p in [first, L) of (p + 1)
        total += (L * (L + 1) - first * (first + 1)) // 2
    return 4 * total * num_q_heads * head_dim

