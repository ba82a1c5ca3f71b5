/*
 * pagedkv.h — C ABI of an MI355X (gfx950) paged KV-cache decode library.
 *
 * The library implements the hot path of PagedAttention decoding: for each sequence
 * of a batch, one new query token attends over that sequence's keys and values,
 * which live in fixed-size physical blocks scattered through a shared pool and are
 * found through a per-sequence block table; a companion call writes each new
 * token's key and value into its slot first.
 *
 * Sources (page title, section):
 *  - "PagedAttention: Treating KV Memory Like Virtual Memory", "How the kernel reads
 *    a block table": address = block_table[i / B] * block stride + (i mod B) * slot
 *    stride; the kernel walks the history tile by tile with a running max and sum.
 *  - "Why AI servers waste memory, and how paging fixes it", "The idea: a block
 *    table" (position p lives in block table[p // B], slot p % B), "The real
 *    implementation" (the append writes the token into slot `offset` of the last
 *    block; a call that cannot succeed changes nothing), "Reading through the table"
 *    (only the first `valid` slots of the last block are read).
 *  - "PagedAttention and Virtual Memory Management", section 1 (M_KV closed form),
 *    section 3 (block partitioning, physical block bytes), section 4 (Addr_K/Addr_V,
 *    block-wise online-softmax decode, split across thread blocks with a
 *    cross-block reduction).
 *
 * Conventions shared by every call
 *  - All tensors are caller-owned device buffers (HBM of the current HIP device),
 *    dense row-major, 16-byte aligned.  The library never allocates per call; the
 *    only memory it may own is a pool it was asked to allocate in kv_pool_create.
 *  - Compute calls only enqueue work on the caller's stream (0 = null stream).
 *    There is no host synchronisation and no host read of device data.
 *  - Every argument check runs on the host before anything is enqueued: a call that
 *    returns an error has changed nothing.  A launch failure returns KV_ERR_HIP.
 *  - K and V are stored in the pool's dtype: fp16, bf16, or FP8 E4M3 (one byte per
 *    element; "PagedAttention and Virtual Memory Management", section 1: b = 1 for
 *    FP8).  Queries, attention outputs and the new keys / values given to
 *    reshape_and_cache use the pool's io_dtype (fp16 or bf16; for 16-bit pools it is
 *    the pool's dtype).  Arithmetic: stored values are widened exactly; dot products and
 *    the softmax are fp32; the softmax weights enter the P.V product on the matrix cores
 *    as 16-bit operands, each weight split into a rounded part and its rounded remainder
 *    (about 16 significand bits; prefill with fp16 io uses one fp16 part, 11 bits), with
 *    the products accumulated in fp32; the output is rounded to the io type with
 *    round-to-nearest-even.
 *  - FP8 E4M3: 1 sign, 4 exponent (bias 7) and 3 mantissa bits, no infinities,
 *    S.1111.111 is NaN, largest finite magnitude 448, no scale factor.  The cache write
 *    rounds to the nearest code (ties to even), saturates larger magnitudes and
 *    infinities to +-448 and writes NaN as S.1111.111.
 *  - Results depend only on logical token positions: the output is bit-identical
 *    under any relabelling of physical blocks, and run-to-run deterministic.
 *  - Device data is trusted on the fast path: block ids past a sequence's length are
 *    never read, an id outside the pool reads as zeros, a length past the table is
 *    clamped, a negative or out-of-range slot writes nothing, and duplicate slots give
 *    an unspecified one of the values.  Checked mode (environment PAGEDKV_CHECK=1, read
 *    per call) validates on the device first, then waits for the stream and returns
 *    KV_ERR_INVALID_ARG, with nothing written, if a used table entry names no block of
 *    the pool, a length lies outside [0, max_blocks * block_size], a slot is out of
 *    range or repeated (reshape_and_cache; for the decode calls that write the new
 *    tokens, the slots of position L - 1), or query offsets are decreasing or a chunk
 *    exceeds max_query_len (paged_attention_prefill).  It synchronises, so it is for
 *    debugging: it is not meant for graph capture, and on its first use per device it
 *    allocates a small status buffer (and a slot bitmap) that lives until the process
 *    ends.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kv_dtype {
    KV_DTYPE_F16 = 0,
    KV_DTYPE_BF16 = 1,
    KV_DTYPE_FP8_E4M3 = 2      /* pool storage only */
} kv_dtype_t;

typedef enum kv_status {
    KV_OK = 0,
    KV_ERR_INVALID_ARG = 1,    /* null pointer, negative size, layer out of range, misalignment */
    KV_ERR_UNSUPPORTED = 2,    /* shape / dtype the kernels are not built for */
    KV_ERR_WORKSPACE = 3,      /* workspace missing or smaller than required */
    KV_ERR_OUT_OF_MEMORY = 4,  /* the pool allocation in kv_pool_create failed */
    KV_ERR_HIP = 5,            /* a HIP runtime call or kernel launch failed */
    KV_ERR_OUT_OF_BLOCKS = 6   /* the block manager has no free block for an append */
} kv_status_t;

/* Geometry of a KV pool.  Supported: block_size 8, 16, 32 or 64 ("PagedAttention and
 * Virtual Memory Management", section 3: B is typically 8, 16 or 32; 16 is the usual
 * default), head_dim 64 or 128, dtype KV_DTYPE_F16 / KV_DTYPE_BF16 / KV_DTYPE_FP8_E4M3,
 * num_blocks >= 1, num_kv_heads >= 1.  io_dtype: KV_DTYPE_F16 or KV_DTYPE_BF16 for an
 * FP8 pool; ignored (taken as dtype) for a 16-bit pool. */
typedef struct kv_pool_desc {
    int32_t num_layers;
    int32_t num_blocks;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t dtype;             /* kv_dtype_t: storage of K and V */
    int32_t io_dtype;          /* kv_dtype_t: queries, outputs, new keys / values */
} kv_pool_desc_t;

/* Opaque, immutable after creation: safe to use from several streams at once. */
typedef struct kv_pool kv_pool_t;

/* Human-readable name of a status code (static string). */
const char* kv_status_string(kv_status_t status);

/* Bytes of K+V per token over all layers, 2 * N_L * N_KV * d_h * b, b = 2 for fp16 /
 * bf16 and 1 for FP8 ("PagedAttention and Virtual Memory Management", section 1,
 * M_KV(L) at L = 1).
 * Returns 0 for an invalid or unsupported descriptor. */
size_t kv_bytes_per_token(const kv_pool_desc_t* desc);

/* Bytes of the whole pool: kv_bytes_per_token * num_blocks * block_size.
 * Memory layout (per layer l, for K then V):
 *   base + (2*l + 0) * S  : K cache [num_blocks][block_size][num_kv_heads][head_dim]
 *   base + (2*l + 1) * S  : V cache, same shape
 * with S = num_blocks * block_size * num_kv_heads * head_dim * b bytes.  Token row
 * (block, offset) of one layer's K is contiguous (num_kv_heads * head_dim elements),
 * so a whole block of one layer is one contiguous stretch.  Returns 0 if invalid. */
size_t kv_pool_bytes(const kv_pool_desc_t* desc);

/* Create a pool handle.
 *  device_base == NULL : the library hipMallocs kv_pool_bytes(desc) bytes on the
 *                        current device and frees them in kv_pool_destroy.
 *  device_base != NULL : the caller's device memory is borrowed (never freed by the
 *                        library); it must be 256-byte aligned and base_bytes must be
 *                        >= kv_pool_bytes(desc).
 * The pool contents are not initialised.  On error *out is left unchanged.
 * Errors: KV_ERR_INVALID_ARG (null desc/out, bad sizes, misaligned or short base),
 * KV_ERR_UNSUPPORTED (block_size, head_dim or dtype), KV_ERR_OUT_OF_MEMORY. */
kv_status_t kv_pool_create(const kv_pool_desc_t* desc, void* device_base, size_t base_bytes,
                           kv_pool_t** out);

/* A pool in pinned host memory with the same layout as a device pool: the "auxiliary
 * physical block pool in CPU host memory" that swapped-out blocks go to ("PagedAttention
 * and Virtual Memory Management", section 6, swapping policy).  Only kv_swap_blocks,
 * kv_pool_get_desc, kv_pool_layer_ptrs (host addresses) and kv_pool_destroy accept it;
 * the attention and cache-write calls return KV_ERR_INVALID_ARG for it.
 *  host_base == NULL : the library allocates kv_pool_bytes(desc) bytes of pinned,
 *                      device-mapped host memory (hipHostMalloc) and frees it in
 *                      kv_pool_destroy.
 *  host_base != NULL : the caller's pinned host memory (allocated pinned, e.g.
 *                      hipHostMalloc), borrowed; 256-byte aligned, base_bytes >=
 *                      kv_pool_bytes(desc); KV_ERR_INVALID_ARG if HIP does not know it
 *                      as host memory mapped for the current device.
 * The contents are not initialised. */
kv_status_t kv_host_pool_create(const kv_pool_desc_t* desc, void* host_base, size_t base_bytes,
                                kv_pool_t** out);

/* 1 if the pool lives in host memory (kv_host_pool_create), 0 if on the device, -1 for
 * NULL. */
int32_t kv_pool_is_host(const kv_pool_t* pool);

/* Destroy a handle; frees the pool memory only if the library allocated it (the pool is
 * cut into blocks once and lives as long as the engine: "Why AI servers waste memory, and
 * how paging fixes it", "The idea: a block table").  NULL is accepted and ignored.  The
 * caller must ensure no enqueued work still uses it. */
kv_status_t kv_pool_destroy(kv_pool_t* pool);

/* Copy the pool's descriptor into *desc (the geometry of "PagedAttention and Virtual
 * Memory Management", section 3: block size, heads, head size, element bytes). */
kv_status_t kv_pool_get_desc(const kv_pool_t* pool, kv_pool_desc_t* desc);

/* Device addresses of layer `layer`'s K and V caches (either output may be NULL): the
 * per-layer pool bases PoolPtr_K and PoolPtr_V of "PagedAttention and Virtual Memory
 * Management", section 4 (Addr_K / Addr_V), laid out as kv_pool_bytes states. */
kv_status_t kv_pool_layer_ptrs(const kv_pool_t* pool, int32_t layer, void** k_cache,
                               void** v_cache);

/* Write new tokens' keys and values into their slots of layer `layer`.
 *  key, value   : [num_tokens][num_kv_heads][head_dim], io dtype.  For an FP8 pool each
 *                 element is rounded to E4M3 as stated above; otherwise the write is a
 *                 bit copy.
 *  slot_mapping : [num_tokens] int64, slot = physical_block * block_size + offset
 *                 ("Why AI servers waste memory, and how paging fixes it", "The idea:
 *                 a block table"; "2.1 PagedAttention", section 5: physical block
 *                 number and offset).  A negative slot means "no write" (padding);
 *                 slots >= num_blocks * block_size are also skipped.  Slots must be
 *                 pairwise distinct; if two tokens name the same slot, which one
 *                 lands is unspecified.
 * The write is ordered before later work on the same stream, so a
 * paged_attention_decode enqueued after it on that stream reads the new tokens.
 * num_tokens == 0 is a no-op. */
kv_status_t reshape_and_cache(kv_pool_t* pool, int32_t layer, const void* key, const void* value,
                              const int64_t* slot_mapping, int32_t num_tokens, hipStream_t stream);

/* Workspace bytes paged_attention_decode needs for this batch shape: the intermediate
 * (m, l, O) that each thread block of a split sequence leaves for the cross-block
 * reduction ("PagedAttention and Virtual Memory Management", section 4), in fp32 --
 * running max, running sum and unnormalised accumulator -- of every (sequence, query
 * head, partition).  0 when no sequence can have more than one partition (then workspace
 * may be NULL).  partition_size 0 means 512.  block_size (the pool's) fixes how many
 * partitions max_blocks_per_seq blocks can hold.
 * Returns SIZE_MAX for invalid arguments. */
size_t paged_attention_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                       int32_t max_blocks_per_seq, int32_t block_size,
                                       int32_t partition_size);

/* Decode attention for one layer.
 *  out          : [batch][num_q_heads][head_dim], io dtype (written).
 *  query        : [batch][num_q_heads][head_dim], io dtype.
 *  block_tables : [batch][max_blocks_per_seq] int32; entry j of row b is the physical
 *                 block holding tokens [Bj, Bj+B) of sequence b (B = the pool's
 *                 block_size).  Entries at or past ceil(context_lens[b] / B) are never
 *                 read (may hold -1).
 *  context_lens : [batch] int32, number of tokens of each sequence, including a token
 *                 just written by reshape_and_cache.  Values are clamped to
 *                 [0, max_blocks_per_seq * B]; a sequence of length 0 gets a zero
 *                 output.  Slots at or past the length in the last block are never read.
 *  num_q_heads  : multiple of the pool's num_kv_heads; query head h reads KV head
 *                 h / (num_q_heads / num_kv_heads) (contiguous GQA groups); group
 *                 sizes 1..16 are supported.
 *  scale        : multiplies q.k before the softmax (normally 1/sqrt(head_dim)).
 *  partition_size: tokens per split-context partition (a multiple of B, at most 4096
 *                 and at most 2048 when B = 8; 0 = 512; larger values return
 *                 KV_ERR_UNSUPPORTED).  A sequence
 *                 longer than one partition is split into partitions processed in
 *                 parallel, whose partial results are combined with the cross-block
 *                 rule ("PagedAttention and Virtual Memory Management", section 4,
 *                 cross-block reduction): inside the partition kernel, through LDS,
 *                 when one work-group holds all of a sequence's partitions, otherwise
 *                 by a second kernel over partial results in the workspace.  When
 *                 work-groups hold whole sequences and the batch needs several rounds of
 *                 them, a one-work-group kernel first writes the sequences' order by
 *                 length, longest first, to the start of the workspace, and the
 *                 work-groups take the sequences in that order (so the longest do not
 *                 start last); the results do not depend on the order.
 *  workspace    : >= paged_attention_workspace_bytes(...) bytes of device memory,
 *                 256-byte aligned (else KV_ERR_INVALID_ARG); contents on entry do not
 *                 matter.
 * Table entries outside [0, num_blocks) for blocks a sequence uses are skipped (the
 * output is then meaningless but no memory outside the pool is read).
 * Errors: KV_ERR_INVALID_ARG, KV_ERR_UNSUPPORTED (group size), KV_ERR_WORKSPACE,
 * KV_ERR_HIP.  batch == 0 is a no-op. */
kv_status_t paged_attention_decode(const kv_pool_t* pool, int32_t layer, void* out,
                                   const void* query, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* context_lens,
                                   int32_t batch, int32_t num_q_heads, float scale,
                                   int32_t partition_size, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* One decode step with the cache write folded in: new_key[b] and new_value[b]
 * ([batch][num_kv_heads][head_dim], io dtype, 16-byte aligned) are the key and value of
 * the token at position context_lens[b] - 1 of sequence b; each is written (rounded to
 * E4M3 for an FP8 pool) into the slot that position has through the table, block
 * table[b][(L-1) / B], offset (L-1) mod B, and then attention runs as in
 * paged_attention_decode.  This is reshape_and_cache with slot_mapping[b] taken from the
 * table, followed by paged_attention_decode, in fewer launches: the matrix-core kernel
 * writes each new row from the wave that then reads it ("Why AI servers waste memory,
 * and how paging fixes it", "The real implementation": the append writes slot `offset`
 * of the last block, then the token is read through the table).  A sequence of length 0,
 * or whose table entry for position L - 1 names no block of the pool, writes nothing.
 * The slots of position L - 1 must be pairwise distinct over the batch, as for
 * reshape_and_cache: a block that several sequences share (before its copy-on-write
 * copy, kv_copy_blocks) may hold the new token of at most one of them, else the result
 * is undefined.
 * Same arguments, results and errors as paged_attention_decode otherwise; the pool's
 * bytes after the call equal those after reshape_and_cache with that slot mapping. */
kv_status_t paged_attention_decode_append(const kv_pool_t* pool, int32_t layer, void* out,
                                          const void* query, const void* new_key,
                                          const void* new_value, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                                          int32_t batch, int32_t num_q_heads, float scale,
                                          int32_t partition_size, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream);

/* The two phases of paged_attention_decode, for callers that time or schedule them
 * separately; same arguments.  paged_attention_partitions writes the final output of
 * every sequence whose partitions it could combine by itself and partial results for
 * the others; paged_attention_reduce combines those partials into `out` (and enqueues
 * nothing when there are none).  Enqueueing partitions then reduce on one stream is
 * exactly paged_attention_decode. */
kv_status_t paged_attention_partitions(const kv_pool_t* pool, int32_t layer, void* out,
                                       const void* query, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                                       int32_t batch, int32_t num_q_heads, float scale,
                                       int32_t partition_size, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);
/* The first phase of paged_attention_decode_append (write the new tokens, partitions);
 * paged_attention_reduce is its second phase. */
kv_status_t paged_attention_partitions_append(const kv_pool_t* pool, int32_t layer, void* out,
                                              const void* query, const void* new_key,
                                              const void* new_value, const int32_t* block_tables,
                                              int32_t max_blocks_per_seq,
                                              const int32_t* context_lens, int32_t batch,
                                              int32_t num_q_heads, float scale,
                                              int32_t partition_size, void* workspace,
                                              size_t workspace_bytes, hipStream_t stream);
kv_status_t paged_attention_reduce(const kv_pool_t* pool, int32_t layer, void* out,
                                   const void* query, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* context_lens,
                                   int32_t batch, int32_t num_q_heads, float scale,
                                   int32_t partition_size, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* Decode attention for a batch whose sequences begin with the same blocks: sequences
 * forked from one prompt, or requests that found one cached prefix ("Why AI servers
 * waste memory, and how paging fixes it", "Sharing a prefix with copy-on-write": forked
 * sequences point at the prompt's blocks until they write; "PagedAttention: Treating KV
 * Memory Like Virtual Memory", "A separate mechanism: automatic prefix caching").  The
 * result is that of paged_attention_decode (or _append, with new_key / new_value) on the
 * same arguments, up to rounding: the same attention over each sequence's whole
 * context, summed in another order.
 *  prefix_blocks : the first prefix_blocks entries of every table row are row 0's (the
 *                  caller, who forked the sequences, knows this count; it is not looked
 *                  for).  0 runs paged_attention_decode(_append) itself.
 * The shared keys are read once for the whole batch instead of once per sequence: the
 * batch's query rows of each KV head form one dense tile against the prefix's keys
 * (matrix cores; the prefix is split over work-groups), each sequence's remaining blocks
 * go through the decode kernels, and the two sets of partial results (m, l, O) are
 * combined per (sequence, query head) with the cross-block rule ("PagedAttention and
 * Virtual Memory Management", section 4), deterministically.  When the table entries
 * after the prefix hold at most max(partition_size, 1,024) tokens, each sequence's
 * remaining blocks are one partition and the decode kernel combines and writes the
 * output itself (two launches); otherwise a third kernel combines the partial results
 * (and so always with PAGEDKV_CASCADE_FUSE=0).
 * Preconditions (checked in checked mode, PAGEDKV_CHECK=1; otherwise the output is
 * undefined if they fail, and nothing outside the pool is read): a row's entries among
 * the first prefix_blocks that its length uses equal row 0's; with new tokens, every
 * sequence of length L > 0 has L > prefix_blocks * B (the token goes into a block of
 * its own, never into a shared one) and prefix_blocks < max_blocks_per_seq.  A sequence
 * shorter than the prefix attends over its own length of it.
 *  workspace : >= paged_attention_shared_prefix_workspace_bytes(...) bytes, 256-byte
 *              aligned; contents on entry do not matter.
 * Other arguments, errors and the cache write as paged_attention_decode_append
 * (new_key and new_value both NULL: no write, as paged_attention_decode). */
kv_status_t paged_attention_decode_shared_prefix(const kv_pool_t* pool, int32_t layer, void* out,
                                                 const void* query, const void* new_key,
                                                 const void* new_value, const int32_t* block_tables,
                                                 int32_t max_blocks_per_seq,
                                                 const int32_t* context_lens, int32_t batch,
                                                 int32_t num_q_heads, float scale,
                                                 int32_t prefix_blocks, int32_t partition_size,
                                                 void* workspace, size_t workspace_bytes,
                                                 hipStream_t stream);
/* The largest prefix_blocks that paged_attention_decode_shared_prefix accepts for these
 * tables (host arrays, as kv_bm_export and kv_pc_export fill them): the number of leading
 * entries of row 0 that are blocks (>= 0) and that every other sequence has too, where a
 * sequence is held only to the entries its length uses (ceil(L / B); a shorter sequence
 * sees its own part of the prefix).  With appending != 0, also at most (L - 1) / B for
 * every sequence of length L > 0: its new token must fall after the prefix, in a block
 * of its own (copy-on-write keeps the written block private; "Why AI servers waste
 * memory, and how paging fixes it", "Sharing a prefix with copy-on-write").
 *  tables  : [batch][max_blocks] int32; lengths: [batch] int32 (clamped to the table).
 * Returns the count, 0 when nothing is shared, or -1 for invalid arguments (null
 * pointers, batch < 1, max_blocks < 1, block_size not 8, 16, 32 or 64).  Reads only the
 * arrays; nothing is enqueued. */
int32_t kv_shared_prefix_blocks(const int32_t* tables, const int32_t* lengths, int32_t batch,
                                int32_t max_blocks, int32_t block_size, int32_t appending);

/* Workspace bytes of paged_attention_decode_shared_prefix for this shape on the current
 * device (the prefix's split follows the device's size): the prefix's partial results
 * (m, l and a scale in fp32, O as 16-bit integers times that scale, for every (sequence,
 * query head, split)), then, when the combine takes a kernel of its own, the suffixes'
 * partial results (as paged_attention_workspace_bytes, for the entries after the prefix,
 * with one partition counted too).  With prefix_blocks == 0,
 * paged_attention_workspace_bytes.
 * SIZE_MAX for invalid arguments (null or host pool, sizes out of range). */
size_t paged_attention_shared_prefix_workspace_bytes(const kv_pool_t* pool, int32_t batch,
                                                     int32_t num_q_heads, int32_t max_blocks_per_seq,
                                                     int32_t prefix_blocks, int32_t partition_size);

/* A batch order for a decode step whose sequences differ in length: the indices of
 * `lengths` (host array, [batch] int32) sorted by length, longest first, equal lengths in
 * batch order, written to `order` (host, [batch] int32).  Most launch plans take their
 * work in batch order (large batches of whole sequences per work-group order themselves,
 * see paged_attention_decode), so a batch built in this order (queries, tables, lengths
 * and outputs permuted alike) leaves the shortest work for the end of the launch, when
 * the GPU is draining.  A scheduling aid for callers that build the batch, not an
 * operation the pages define; the attention's result per sequence does not depend on the
 * order.  Returns 0, or -1 for null pointers or batch < 0.  Reads and writes host memory
 * only. */
int32_t kv_decode_order(const int32_t* lengths, int32_t batch, int32_t* order);

/* Bytes of the scratch array the library keeps on each GPU for
 * paged_attention_decode_noalloc (64 MiB). */
#define PAGEDKV_SCRATCH_BYTES ((size_t)64 << 20)

/* paged_attention_decode for callers that cannot allocate memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same arguments
 * without the workspace, the same kernels and the same output bits.  The fp32 partial
 * results go to a scratch array of PAGEDKV_SCRATCH_BYTES that the library keeps in device
 * memory, one per GPU, from the library's load until the process ends; the call itself
 * allocates nothing.  Its device address is looked up on the first call on each device
 * (that call must run with the device current, as every call must).
 *  - The shape must need at most PAGEDKV_SCRATCH_BYTES of workspace
 *    (paged_attention_workspace_bytes(...) <= PAGEDKV_SCRATCH_BYTES), else the call
 *    returns KV_ERR_WORKSPACE and enqueues nothing.  For example 64 sequences x 8,192
 *    tokens with 32 query heads of 128 need 17 MB; 512 sequences x 4,096 tokens with 64
 *    heads of 128 need 136 MB and are refused.
 *  - Every call on one GPU shares that GPU's array and leaves its partial results in it.
 *    Nothing in it needs to start at zero.  Calls that overlap in time on one GPU (on
 *    different streams, or from several threads without ordering) race on the array and
 *    give undefined results: serialise them, e.g. on one stream.
 *  - Checked mode (PAGEDKV_CHECK) does not apply: its passes allocate and synchronise.
 * Errors: as paged_attention_decode, with KV_ERR_WORKSPACE for a shape beyond the array
 * and KV_ERR_HIP if the array's address cannot be found. */
kv_status_t paged_attention_decode_noalloc(const kv_pool_t* pool, int32_t layer, void* out,
                                           const void* query, const int32_t* block_tables,
                                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                                           int32_t batch, int32_t num_q_heads, float scale,
                                           int32_t partition_size, hipStream_t stream);

/* Copy-on-write copies on the device, for every layer of the pool, K and V:
 *  copies : [num_copies][3] int32 device array of (src, dst, rows); the first `rows`
 *           token rows of physical block src are copied into block dst and the other
 *           rows of dst are left as they are ("PagedAttention and Virtual Memory
 *           Management", section 5, case 2: the o rows already in the shared block go
 *           to the new block before the new token is written into slot o).
 * kv_bm_append produces these triples.  Blocks named as dst must be distinct and not be
 * the src of another triple of the same call (then the copies are independent; the
 * manager's triples always are).  Enqueue it before the reshape_and_cache of the same
 * step.  A triple with a block outside [0, num_blocks), rows outside [0, block_size] or
 * src == dst is skipped on the device.  num_copies == 0 is a no-op.
 * Errors: KV_ERR_INVALID_ARG (null pool or copies, negative count, copies not 4-byte
 * aligned), KV_ERR_HIP. */
kv_status_t kv_copy_blocks(kv_pool_t* pool, const int32_t* copies, int32_t num_copies,
                           hipStream_t stream);

/* Swap copies: for every pair (src block, dst block) of pairs[0..num_pairs), all B rows
 * of block src of every layer's K and V in pool src are copied to block dst of pool dst
 * ("PagedAttention and Virtual Memory Management", section 6, swapping policy: device
 * to host on preemption, host to device on resume).  The pools have the same
 * num_layers, block_size, num_kv_heads, head_dim and dtype (num_blocks may differ); one
 * or both may be host pools.  Bytes are copied unchanged.
 *  pairs : [num_pairs][2] int32 in device memory (or pinned host memory), as
 *          kv_bm_move writes them.  Destination blocks must be distinct; a pair naming a
 *          block outside its pool is skipped.  src and dst must not be the same pool.
 * One kernel launch on `stream`, asynchronous: the caller keeps the pairs and both
 * pools alive until the stream reaches it.  The kernel runs on a fixed number of
 * work-groups (far fewer than the CUs) so decode kernels on other streams keep the
 * rest of the chip.
 * Errors: KV_ERR_INVALID_ARG (null or equal pools, shapes that differ, num_pairs < 0,
 * null or misaligned pairs), KV_ERR_HIP (launch failed). */
kv_status_t kv_swap_blocks(const kv_pool_t* src, kv_pool_t* dst, const int32_t* pairs,
                           int32_t num_pairs, hipStream_t stream);

/* ------------------------------------------------------------------ block manager
 * Host-side bookkeeping that decides where tokens go: a free list of physical blocks,
 * a reference count per block and a block table per request ("Why AI servers waste
 * memory, and how paging fixes it": "The idea: a block table", "A hand-worked
 * example", "The real implementation", "Sharing a prefix with copy-on-write";
 * "PagedAttention and Virtual Memory Management", section 5).
 *  - New blocks come from the front of the free list; freed blocks join its back.
 *  - Request ids are the caller's 64-bit integers.
 *  - Every call checks all it needs before changing anything: a call that returns an
 *    error has changed nothing.
 *  - Host memory only; all array arguments are host arrays.  Not thread-safe.
 * One decode step with a pool: kv_bm_append (slots + copies) -> copy both to the device
 * -> kv_copy_blocks -> reshape_and_cache -> kv_bm_export (tables, lengths) -> copy to
 * the device -> paged_attention_decode. */
typedef struct kv_block_manager kv_block_manager_t;

/* A manager of num_blocks blocks of block_size token slots (any size >= 1; a pool used
 * with it has the same block_size).  The free list starts as 0, 1, ..., num_blocks - 1. */
kv_status_t kv_bm_create(int32_t num_blocks, int32_t block_size, kv_block_manager_t** out);
kv_status_t kv_bm_destroy(kv_block_manager_t* bm);

/* A new request with an empty table.  KV_ERR_INVALID_ARG if the id exists. */
kv_status_t kv_bm_add_request(kv_block_manager_t* bm, int64_t rid);

/* child starts as a copy of parent's table and length, and every block the table names
 * gains one reference; nothing is allocated or copied.  Forking k - 1 children adds
 * k - 1 to each block ("PagedAttention and Virtual Memory Management", section 5).
 * KV_ERR_INVALID_ARG if parent is unknown or child exists. */
kv_status_t kv_bm_fork(kv_block_manager_t* bm, int64_t parent, int64_t child);

/* Drop the request: each block of its table loses one reference, front to back, and a
 * block nobody names any more joins the back of the free list.  Its contents stay. */
kv_status_t kv_bm_free_request(kv_block_manager_t* bm, int64_t rid);

/* Reserve slots for counts[i] new tokens of request rids[i], request after request in
 * the order given (counts == NULL: one token each, a decode step).
 *  slots  : [sum counts] int64 out, slot = physical block * block_size + offset, in order.
 *  copies : [n][3] int32 out (room for n triples), *num_copies set: (src, dst, rows) for
 *           each append whose last block was shared and had room -- it got a new block
 *           and the rows already written must be copied (kv_copy_blocks).
 * A token at a block boundary takes a new block from the free list.
 * All or nothing: KV_ERR_OUT_OF_BLOCKS if the free list cannot cover the whole batch,
 * KV_ERR_INVALID_ARG for an unknown id, a negative count or buffers that are too small;
 * in both cases nothing changed. */
kv_status_t kv_bm_append(kv_block_manager_t* bm, const int64_t* rids, const int32_t* counts,
                         int32_t n, int64_t* slots, int64_t slots_cap, int32_t* copies,
                         int32_t copies_cap, int32_t* num_copies);

/* Views. */
kv_status_t kv_bm_get_length(const kv_block_manager_t* bm, int64_t rid, int32_t* length);
kv_status_t kv_bm_get_table(const kv_block_manager_t* bm, int64_t rid, int32_t* table,
                            int32_t cap, int32_t* num);
/* Block tables and lengths of rids[0..n) in the layout paged_attention_decode reads:
 * tables [n][max_blocks] int32, padded with -1; lengths [n] int32.  KV_ERR_INVALID_ARG
 * if an id is unknown or a table is longer than max_blocks (then nothing is written). */
kv_status_t kv_bm_export(const kv_block_manager_t* bm, const int64_t* rids, int32_t n,
                         int32_t max_blocks, int32_t* tables, int32_t* lengths);
/* Number of free blocks (-1 for a null manager). */
int32_t kv_bm_num_free(const kv_block_manager_t* bm);
kv_status_t kv_bm_ref_count(const kv_block_manager_t* bm, int32_t block, int32_t* count);
/* The free list, front first. */
kv_status_t kv_bm_free_list(const kv_block_manager_t* bm, int32_t* blocks, int32_t cap,
                            int32_t* num);

/* Swap: move requests rids[0..n) from manager src to manager dst -- out to a manager of
 * host blocks, or back in to the device's ("PagedAttention and Virtual Memory
 * Management", section 6, swapping policy: the victim's blocks go to a block pool in
 * host memory, the GPU blocks return to the free list, and on resume they come back).
 * Every distinct block the moved tables name gets one block of dst, taken from the
 * front of dst's free list in first-seen order (requests in the order given, tables
 * front to back); blocks the moved requests share stay shared in dst with the same
 * counts.  Then src drops the requests as kv_bm_free_request does.  A block that a
 * request left in src still names keeps its references there (its copy goes along).
 *  pairs : [*num_pairs][2] int32 out, (src block, dst block) in first-seen order -- the
 *          copies kv_swap_blocks must make.  pairs_cap >= the total table length of the
 *          moved requests is always enough.
 * All or nothing: KV_ERR_OUT_OF_BLOCKS if dst's free list is shorter than the distinct
 * blocks; KV_ERR_INVALID_ARG for an unknown or repeated id, an id dst already has,
 * different block sizes, src == dst or too small a pairs buffer; nothing changes. */
kv_status_t kv_bm_move(kv_block_manager_t* src, kv_block_manager_t* dst, const int64_t* rids,
                       int32_t n, int32_t* pairs, int32_t pairs_cap, int32_t* num_pairs);

/* Multi-token (prefill / chunked-prefill) attention for one layer: each sequence has a
 * chunk of new tokens whose keys and values are already in the pool (reshape_and_cache),
 * and each of them attends causally over the sequence's paged keys and values
 * ("PagedAttention: Treating KV Memory Like Virtual Memory", section "What the allocator
 * actually sees": besides one-token decode steps a request arrives as a prompt processed
 * in parallel, or in pieces cut to a step's token budget; "PagedAttention and Virtual
 * Memory Management": the prefill phase processes the prompt in parallel).
 *  query, out   : [T][num_q_heads][head_dim], io dtype; the chunks of all sequences packed
 *                 one after another.
 *  query_start  : [batch + 1] int32 device, non-decreasing, query_start[0] = 0: sequence
 *                 b's queries are rows [query_start[b], query_start[b+1]), n_b of them.
 *  max_query_len: an upper bound on every n_b (host value; sizes the launch).  Queries
 *                 past it are not computed.
 *  context_lens : [batch] int32, length L_b including the chunk: query i of sequence b is
 *                 at position p = L_b - n_b + i and reads positions [0, p].  A query with
 *                 p < 0 gets a zero output.
 *  block_tables, max_blocks_per_seq, num_q_heads, scale: as for paged_attention_decode.
 * Arithmetic as in decode (fp32 scores, softmax and accumulation; the output rounded to
 * the io dtype).  No workspace.  Errors: KV_ERR_INVALID_ARG, KV_ERR_UNSUPPORTED (group
 * size), KV_ERR_HIP.  batch == 0 or max_query_len == 0 is a no-op. */
kv_status_t paged_attention_prefill(const kv_pool_t* pool, int32_t layer, void* out,
                                    const void* query, const int32_t* query_start,
                                    int32_t max_query_len, const int32_t* block_tables,
                                    int32_t max_blocks_per_seq, const int32_t* context_lens,
                                    int32_t batch, int32_t num_q_heads, float scale,
                                    hipStream_t stream);

/* paged_attention_prefill for launches too small to fill the GPU (a single prompt with
 * few KV heads, say): each row tile's key range is split over up to 8 work-groups, whose
 * partial results (the per-row running maximum, weight sum and unnormalised weighted sum
 * of values, in fp32) a second kernel combines with the rule that merges split-context
 * partitions ("PagedAttention and Virtual Memory Management", section 4, the reduction
 * across thread blocks).  The split count follows from the arguments below and the
 * current device (its compute units and the kernel's occupancy), so size the workspace
 * with the same device current; with one split the call is paged_attention_prefill (same
 * bits, no workspace used).
 *  num_tokens : rows of query and out (query_start[batch] <= num_tokens); partial
 *               results of rows past it are not written.
 *  workspace  : device memory, 256-byte aligned, of at least
 *               paged_attention_prefill_workspace_bytes(pool, batch, num_q_heads,
 *               num_tokens, max_query_len, max_blocks_per_seq) bytes (0: none needed);
 *               contents on entry do not matter; caller-owned, not retained.
 * Results agree with paged_attention_prefill to rounding (the sums are taken in another
 * order) and are deterministic.  Errors: as paged_attention_prefill, and
 * KV_ERR_WORKSPACE for too small a workspace. */
size_t paged_attention_prefill_workspace_bytes(const kv_pool_t* pool, int32_t batch,
                                               int32_t num_q_heads, int32_t num_tokens,
                                               int32_t max_query_len, int32_t max_blocks_per_seq);
kv_status_t paged_attention_prefill_split(const kv_pool_t* pool, int32_t layer, void* out,
                                          const void* query, const int32_t* query_start,
                                          int32_t max_query_len, int32_t num_tokens,
                                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t batch,
                                          int32_t num_q_heads, float scale, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ prefix cache
 * Host-side automatic prefix caching on a block pool: which physical blocks a new request
 * can reuse because an earlier one computed the same prefix ("PagedAttention: Treating
 * KV Memory Like Virtual Memory", "A separate mechanism: automatic prefix caching"; "2.1
 * PagedAttention", section 9, BlockPool / KVCacheManager).
 *  - A block is hashed when it fills: 64-bit FNV-1a over the little-endian bytes of the
 *    previous block's hash (0 before the first block), the block's token ids (int32) and,
 *    for a request's first block only, the request's 64-bit salt.  The hashes form a
 *    chain, so a hit means agreement from the first token; a match ends on a block
 *    boundary.  A block whose hash is already cached (the same prefix in another block)
 *    stays uncached.
 *  - A hit copies nothing: the block's count rises, and a free cached block leaves the
 *    free queue.  Finishing lowers the counts of the request's blocks, last block first;
 *    blocks that reach zero return to the free queue with their hash, hash-less ones at
 *    the head (reused first, in that order) and cached ones at the tail (evicted last).
 *    Taking a cached free block for new data evicts its hash.
 *  - Every call checks everything before changing anything.  Host memory only; not
 *    thread-safe.  Shared blocks are full, so nothing is ever written into a shared
 *    block and no copy-on-write copy is needed. */
typedef struct kv_prefix_cache kv_prefix_cache_t;

/* num_blocks blocks of block_size token slots; the free queue starts as 0 .. n-1. */
kv_status_t kv_pc_create(int32_t num_blocks, int32_t block_size, kv_prefix_cache_t** out);
kv_status_t kv_pc_destroy(kv_prefix_cache_t* pc);

/* Start request rid with prompt[0..n): the leading full blocks of the prompt found in the
 * cache become its first blocks; *found_tokens is their token count (a multiple of
 * block_size).  The rest of the prompt is added with kv_pc_append.  KV_ERR_INVALID_ARG if
 * rid exists. */
kv_status_t kv_pc_add_request(kv_prefix_cache_t* pc, int64_t rid, const int32_t* prompt,
                              int32_t n, uint64_t salt, int32_t* found_tokens);

/* Slots (block * block_size + offset) for the request's next n tokens, whose ids are
 * tokens[0..n); blocks that fill up are hashed and cached.  KV_ERR_OUT_OF_BLOCKS if the
 * free queue cannot cover them (nothing changed). */
kv_status_t kv_pc_append(kv_prefix_cache_t* pc, int64_t rid, const int32_t* tokens, int32_t n,
                         int64_t* slots, int64_t slots_cap);
/* One decode step: token tokens[i] for request rids[i], i < n, the n requests distinct;
 * slots[i] receives its slot.  The same as kv_pc_append of one token to each request in
 * order, in one call, checked as a whole first: KV_ERR_INVALID_ARG for an unknown or
 * repeated id, KV_ERR_OUT_OF_BLOCKS if the requests whose last block is full need more
 * blocks than are free; nothing changes then.  n == 0 is a no-op. */
kv_status_t kv_pc_append_step(kv_prefix_cache_t* pc, const int64_t* rids, const int32_t* tokens,
                              int32_t n, int64_t* slots);
kv_status_t kv_pc_free_request(kv_prefix_cache_t* pc, int64_t rid);

/* Views. */
kv_status_t kv_pc_get_length(const kv_prefix_cache_t* pc, int64_t rid, int32_t* length);
kv_status_t kv_pc_get_table(const kv_prefix_cache_t* pc, int64_t rid, int32_t* table, int32_t cap,
                            int32_t* num);
/* Tables ([n][max_blocks], -1 padded) and lengths of rids, as paged_attention_* read them. */
kv_status_t kv_pc_export(const kv_prefix_cache_t* pc, const int64_t* rids, int32_t n,
                         int32_t max_blocks, int32_t* tables, int32_t* lengths);
int32_t kv_pc_num_free(const kv_prefix_cache_t* pc);
int32_t kv_pc_num_cached(const kv_prefix_cache_t* pc);
/* The free queue, head first. */
kv_status_t kv_pc_free_queue(const kv_prefix_cache_t* pc, int32_t* blocks, int32_t cap, int32_t* num);
/* Count, cached flag and hash (0 if uncached) of a block; outputs may be NULL. */
kv_status_t kv_pc_block_info(const kv_prefix_cache_t* pc, int32_t block, int32_t* ref_count,
                             int32_t* is_cached, uint64_t* hash);
/* The chain hash of one block (first != 0: the request's first block, salt mixed in). */
uint64_t kv_pc_hash_block(uint64_t prev, const int32_t* tokens, int32_t n, int32_t first,
                          uint64_t salt);

/* Test hook: copy each sequence's K and V, through its block table, into contiguous
 * buffers ("Why AI servers waste memory, and how paging fixes it", "Reading through
 * the table").  k_out, v_out: [batch][max_blocks_per_seq * B][num_kv_heads][head_dim]
 * in the pool's storage dtype; row t of sequence b is the pool row (table[b][t / B],
 * t % B) for t < context_lens[b] and zero otherwise.  Bit copy. */
kv_status_t kv_pool_gather(const kv_pool_t* pool, int32_t layer, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t batch, void* k_out, void* v_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
