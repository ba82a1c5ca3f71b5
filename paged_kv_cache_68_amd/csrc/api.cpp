// C ABI of the paged decode library: argument checks (host only, before anything is
// enqueued), pool bookkeeping and kernel dispatch.  See include/pagedkv.h.

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>

#include <hip/hip_runtime_api.h>

#include "internal.h"

using pkv::ceil_div;

namespace {

constexpr size_t kAlign = 16;

bool aligned(const void* p, size_t a = kAlign) {
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// Bytes per stored K / V element, and the 16-bit type of queries, outputs and new keys.
size_t elem_bytes(const kv_pool_desc_t& d) { return d.dtype == KV_DTYPE_FP8_E4M3 ? 1 : 2; }
int32_t io_dtype(const kv_pool_desc_t& d) { return d.dtype == KV_DTYPE_FP8_E4M3 ? d.io_dtype : d.dtype; }

kv_status_t check_desc(const kv_pool_desc_t* d) {
    if (!d) return KV_ERR_INVALID_ARG;
    if (d->num_layers < 1 || d->num_blocks < 1 || d->num_kv_heads < 1 || d->block_size < 1 ||
        d->head_dim < 1)
        return KV_ERR_INVALID_ARG;
    if (d->block_size != 8 && d->block_size != 16 && d->block_size != 32 && d->block_size != 64)
        return KV_ERR_UNSUPPORTED;
    if (d->head_dim != 64 && d->head_dim != 128) return KV_ERR_UNSUPPORTED;
    if (d->dtype != KV_DTYPE_F16 && d->dtype != KV_DTYPE_BF16 && d->dtype != KV_DTYPE_FP8_E4M3)
        return KV_ERR_UNSUPPORTED;
    if (d->dtype == KV_DTYPE_FP8_E4M3 && d->io_dtype != KV_DTYPE_F16 && d->io_dtype != KV_DTYPE_BF16)
        return KV_ERR_UNSUPPORTED;
    // a layer's cache must be addressable with 64-bit offsets and the slot count with int64
    const unsigned __int128 bytes = static_cast<unsigned __int128>(d->num_blocks) * d->block_size *
                                    d->num_kv_heads * d->head_dim * elem_bytes(*d) * 2u *
                                    d->num_layers;
    if (bytes >> 62) return KV_ERR_INVALID_ARG;
    return KV_OK;
}

size_t cache_bytes(const kv_pool_desc_t* d) {
    return static_cast<size_t>(d->num_blocks) * d->block_size * d->num_kv_heads * d->head_dim *
           elem_bytes(*d);
}

struct DecodeShape {
    int32_t group = 0;
    int32_t part_blocks = 0;
    int32_t num_parts = 0;
    size_t ws_needed = 0;
};

size_t workspace_for(int32_t batch, int32_t hq, int32_t d, int32_t num_parts) {
    if (num_parts <= 1) return 0;
    const size_t n = static_cast<size_t>(batch) * hq * num_parts;
    const size_t acc = n * d * sizeof(float);
    const size_t ml = n * 2 * sizeof(float);
    return ((acc + 255) / 256) * 256 + ml;
}

kv_status_t check_decode(const kv_pool_t* pool, int32_t layer, void* out, const void* query,
                         const int32_t* block_tables, int32_t max_blocks,
                         const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                         float scale, int32_t partition_size, void* workspace,
                         size_t workspace_bytes, DecodeShape* shape, bool check_workspace = true) {
    if (!pool || pool->host) return KV_ERR_INVALID_ARG;
    const kv_pool_desc_t& d = pool->desc;
    if (layer < 0 || layer >= d.num_layers) return KV_ERR_INVALID_ARG;
    if (batch < 0) return KV_ERR_INVALID_ARG;
    if (num_q_heads < 1) return KV_ERR_INVALID_ARG;
    if (num_q_heads % d.num_kv_heads != 0) return KV_ERR_UNSUPPORTED;
    const int32_t group = num_q_heads / d.num_kv_heads;
    if (group > pkv::kMaxGroup) return KV_ERR_UNSUPPORTED;
    if (!(scale == scale)) return KV_ERR_INVALID_ARG;     // NaN scale
    if (partition_size == 0) partition_size = pkv::kDefaultPartition;
    if (partition_size < d.block_size || partition_size % d.block_size != 0)
        return KV_ERR_INVALID_ARG;
    const int32_t tile = d.block_size < pkv::kTile ? d.block_size : pkv::kTile;
    if (partition_size > pkv::kMaxPartition || partition_size > pkv::kMaxTilesPerWave * tile)
        return KV_ERR_UNSUPPORTED;
    if (batch == 0) {
        shape->group = group;
        return KV_OK;
    }
    if (max_blocks < 1) return KV_ERR_INVALID_ARG;
    if (!out || !query || !block_tables || !context_lens) return KV_ERR_INVALID_ARG;
    if (!aligned(out) || !aligned(query) || !aligned(block_tables, 4) || !aligned(context_lens, 4))
        return KV_ERR_INVALID_ARG;
    if (static_cast<int64_t>(max_blocks) * d.block_size > INT32_MAX) return KV_ERR_INVALID_ARG;
    const int32_t part_blocks = partition_size / tile;          // in tiles
    const int32_t num_parts = static_cast<int32_t>(
        ceil_div(static_cast<int64_t>(max_blocks) * d.block_size, partition_size));
    if (static_cast<int64_t>(batch) * d.num_kv_heads * num_parts > INT32_MAX)
        return KV_ERR_INVALID_ARG;
    const size_t need = workspace_for(batch, num_q_heads, d.head_dim, num_parts);
    if (need > 0 && check_workspace) {
        if (!workspace || workspace_bytes < need) return KV_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return KV_ERR_INVALID_ARG;
    }
    shape->group = group;
    shape->part_blocks = part_blocks;
    shape->num_parts = num_parts;
    shape->ws_needed = need;
    return KV_OK;
}

pkv::DecodeArgs make_args(const kv_pool_t* pool, int32_t layer, void* out, const void* query,
                          const int32_t* block_tables, int32_t max_blocks,
                          const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                          float scale, void* workspace, const DecodeShape& s) {
    const kv_pool_desc_t& d = pool->desc;
    pkv::DecodeArgs a;
    char* kc = pool->base + static_cast<size_t>(2 * layer) * pool->cache_bytes;
    a.q = static_cast<const uint16_t*>(query);
    a.k = reinterpret_cast<const uint8_t*>(kc);
    a.v = reinterpret_cast<const uint8_t*>(kc + pool->cache_bytes);
    a.row_bytes = d.num_kv_heads * d.head_dim * static_cast<int32_t>(elem_bytes(d));
    a.tables = block_tables;
    a.lens = context_lens;
    a.out = static_cast<uint16_t*>(out);
    a.new_k = nullptr;
    a.new_v = nullptr;
    const size_t n = static_cast<size_t>(batch) * num_q_heads * s.num_parts;
    a.ws_acc = static_cast<float*>(workspace);
    a.ws_ml = workspace ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                   ((n * d.head_dim * sizeof(float) + 255) / 256) * 256)
                        : nullptr;
    a.batch = batch;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = d.num_kv_heads;
    a.max_blocks = max_blocks;
    a.table_stride = max_blocks;
    a.len_offset = 0;
    a.keep_partials = 0;
    a.pre_acc = nullptr;
    a.pre_ml = nullptr;
    a.pre_parts = 0;
    a.order = nullptr;
    a.num_blocks = d.num_blocks;
    a.block_size = d.block_size;
    a.tile_tokens = d.block_size < pkv::kTile ? d.block_size : pkv::kTile;
    a.tiles_log2 = 0;
    while ((a.tile_tokens << a.tiles_log2) < d.block_size) ++a.tiles_log2;
    a.part_blocks = s.part_blocks;
    a.num_parts = s.num_parts;
    a.scale_log2 = scale * 1.4426950408889634f;
    // PAGEDKV_XCD_CHUNK overrides the chunk of the XCD renumbering (tuning knob; 0 keeps
    // launch order)
    const char* x = getenv("PAGEDKV_XCD_CHUNK");
    a.xcd_chunk = x ? atoi(x) : 16;
    if (a.xcd_chunk < 0) a.xcd_chunk = 0;
    // bytes this call can touch: the sequences' table rows, and never more than the
    // layer's K and V caches; PAGEDKV_STREAM=0/1 overrides the choice
    const size_t block_bytes = static_cast<size_t>(d.block_size) * a.row_bytes * 2;
    const size_t reach = block_bytes * std::min<size_t>(static_cast<size_t>(batch) * max_blocks,
                                                       static_cast<size_t>(d.num_blocks));
    a.streamed = reach > pkv::kStreamThresholdBytes ? 1 : 0;
    a.stream_loads = a.streamed;
    // (a margin below 2 GiB leaves room for an offset that is past the end but still fits)
    a.layer_bytes = pool->cache_bytes <= 0x7FF00000u ? static_cast<int32_t>(pool->cache_bytes) : 0;
    const char* st = getenv("PAGEDKV_STREAM");
    if (st && (st[0] == '0' || st[0] == '1')) a.stream_loads = st[0] - '0';
    return a;
}

// ---- checked mode (PAGEDKV_CHECK=1, read per call): validation pre-passes on the
// caller's stream, then a wait and a read of the status word.  Per device the library
// keeps a status word and a bitmap of slots (grown on demand) until the process ends.
bool checked_mode() {
    const char* e = getenv("PAGEDKV_CHECK");
    return e && e[0] == '1';
}

struct CheckBuffers {
    uint32_t* status = nullptr;
    uint32_t* seen = nullptr;
    int64_t seen_words = 0;
};

std::mutex g_check_mutex;
CheckBuffers g_check[64];

// The device's buffers, with room for `slots` bits; nullptr on failure.
CheckBuffers* check_buffers(int64_t slots) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_check_mutex);
    CheckBuffers& cb = g_check[dev];
    if (!cb.status && hipMalloc(reinterpret_cast<void**>(&cb.status), sizeof(uint32_t)) != hipSuccess) {
        (void)hipGetLastError();
        cb.status = nullptr;
        return nullptr;
    }
    const int64_t words = (slots + 31) / 32;
    if (words > cb.seen_words) {
        if (cb.seen && hipFree(cb.seen) != hipSuccess) (void)hipGetLastError();
        cb.seen = nullptr;
        cb.seen_words = 0;
        if (hipMalloc(reinterpret_cast<void**>(&cb.seen), static_cast<size_t>(words) * 4) != hipSuccess) {
            (void)hipGetLastError();
            cb.seen = nullptr;
            return nullptr;
        }
        cb.seen_words = words;
    }
    return &cb;
}

// Clear the status word, run `launch(status, seen)`, wait, and map the result.
template <class Launch>
kv_status_t run_check(int64_t slots, hipStream_t stream, Launch launch) {
    CheckBuffers* cb = check_buffers(slots);
    if (!cb) return KV_ERR_OUT_OF_MEMORY;
    uint32_t word = 0;
    if (pkv::launch_clear_word(cb->status, stream) != hipSuccess ||
        launch(cb->status, cb->seen) != hipSuccess ||
        hipMemcpyAsync(&word, cb->status, sizeof(word), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess) {
        (void)hipGetLastError();
        return KV_ERR_HIP;
    }
    return word ? KV_ERR_INVALID_ARG : KV_OK;
}

kv_status_t check_tables_on_device(const kv_pool_t* pool, const int32_t* tables, int32_t max_blocks,
                                   const int32_t* lens, int32_t batch, hipStream_t stream) {
    return run_check(0, stream, [&](uint32_t* status, uint32_t*) {
        return pkv::launch_check_tables(tables, max_blocks, lens, batch, pool->desc.num_blocks,
                                        pool->desc.block_size, status, stream);
    });
}

enum Phase { kBoth = 3, kPartitions = 1, kReduce = 2 };

kv_status_t decode_impl(int phases, const kv_pool_t* pool, int32_t layer, void* out,
                        const void* query, const int32_t* block_tables, int32_t max_blocks,
                        const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                        float scale, int32_t partition_size, void* workspace,
                        size_t workspace_bytes, hipStream_t stream,
                        const void* new_key = nullptr, const void* new_value = nullptr,
                        bool allow_checked = true) {
    DecodeShape s;
    kv_status_t st = check_decode(pool, layer, out, query, block_tables, max_blocks, context_lens,
                                  batch, num_q_heads, scale, partition_size, workspace,
                                  workspace_bytes, &s);
    if (st != KV_OK) return st;
    if (batch == 0) return KV_OK;
    if (allow_checked && checked_mode() && (phases & kPartitions)) {
        st = check_tables_on_device(pool, block_tables, max_blocks, context_lens, batch, stream);
        if (st != KV_OK) return st;
        if (new_key) {
            const int64_t slots = static_cast<int64_t>(pool->desc.num_blocks) * pool->desc.block_size;
            st = run_check(slots, stream, [&](uint32_t* status, uint32_t* seen) {
                return pkv::launch_check_append_slots(block_tables, max_blocks, context_lens, batch,
                                                      pool->desc.num_blocks, pool->desc.block_size,
                                                      seen, status, stream);
            });
            if (st != KV_OK) return st;
        }
    }
    pkv::DecodeArgs a = make_args(pool, layer, out, query, block_tables, max_blocks,
                                  context_lens, batch, num_q_heads, scale, workspace, s);
    a.new_k = static_cast<const uint16_t*>(new_key);
    a.new_v = static_cast<const uint16_t*>(new_value);
    if (phases & kPartitions) {
        if (pkv::launch_partitions(pool->desc.dtype, io_dtype(pool->desc), pool->desc.head_dim,
                                   s.group, a, stream) !=
            hipSuccess)
            return KV_ERR_HIP;
    }
    if ((phases & kReduce) && s.num_parts > 1) {
        // the partition kernel may already have merged chunks of partitions
        const int chunk = pkv::partition_chunk(pool->desc.dtype, io_dtype(pool->desc),
                                               pool->desc.head_dim, s.group, a);
        pkv::DecodeArgs r = a;
        r.part_blocks = a.part_blocks * chunk;
        r.num_parts = static_cast<int32_t>(ceil_div(a.num_parts, chunk));
        if (r.num_parts > 1 &&
            pkv::launch_reduce(io_dtype(pool->desc), pool->desc.head_dim, r, stream) != hipSuccess)
            return KV_ERR_HIP;
    }
    return KV_OK;
}

// The launch shape of a prefill call (host values only): waves per work-group, row tiles
// per (sequence, KV head) and, for the split entry point, work-groups per row tile.
struct PrefillPlan {
    int32_t group = 0;
    int waves = 4;
    int64_t row_tiles = 0;
    int splits = 1;
};

kv_status_t plan_prefill(const kv_pool_t* pool, int32_t batch, int32_t num_q_heads,
                         int32_t max_query_len, int32_t max_blocks_per_seq, bool may_split,
                         PrefillPlan* pl) {
    const kv_pool_desc_t& d = pool->desc;
    if (num_q_heads % d.num_kv_heads != 0) return KV_ERR_UNSUPPORTED;
    pl->group = num_q_heads / d.num_kv_heads;
    if (pl->group > pkv::kMaxGroup) return KV_ERR_UNSUPPORTED;
    const int64_t rows = static_cast<int64_t>(max_query_len) * pl->group;
    pl->waves = pkv::prefill_waves_for(static_cast<int64_t>(batch) * d.num_kv_heads, rows);
    pl->row_tiles = ceil_div(rows, 32 * pl->waves);
    pl->splits = 1;
    if (!may_split || max_query_len == 0 || batch == 0) return KV_OK;
    // split the key range when the row tiles leave resident work-groups idle: enough
    // splits to fill them, at most kMaxPrefillSplits, and at least 4 stages of 64 keys each
    const int64_t wgs = static_cast<int64_t>(batch) * d.num_kv_heads * pl->row_tiles;
    int64_t resident = pkv::prefill_resident_groups(d.dtype, io_dtype(d), d.head_dim, pl->waves);
    if (resident <= 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
            (void)hipGetLastError();
            cus = 256;
        }
        resident = 2 * static_cast<int64_t>(cus);     // no occupancy known: two per CU
    }
    const int64_t max_stages = ceil_div(static_cast<int64_t>(max_blocks_per_seq) * d.block_size, 64);
    int64_t splits = wgs < resident ? ceil_div(resident, wgs) : 1;
    splits = std::min<int64_t>({splits, pkv::kMaxPrefillSplits, std::max<int64_t>(1, max_stages / 4)});
    const char* e = getenv("PAGEDKV_PREFILL_SPLITS");
    if (e && atoi(e) >= 1) splits = std::min(atoi(e), pkv::kMaxPrefillSplits);
    pl->splits = static_cast<int>(splits);
    return KV_OK;
}

// bytes of the partial results: acc then (m, l), each 256-byte aligned
size_t prefill_partial_bytes(int32_t num_tokens, int32_t num_q_heads, int32_t head_dim, int splits,
                             size_t* ml_offset) {
    const size_t parts = static_cast<size_t>(num_tokens) * num_q_heads * splits;
    const size_t acc = (parts * head_dim * 4 + 255) & ~size_t(255);
    if (ml_offset) *ml_offset = acc;
    return acc + ((parts * 8 + 255) & ~size_t(255));
}

kv_status_t prefill_impl(const kv_pool_t* pool, int32_t layer, void* out, const void* query,
                         const int32_t* query_start, int32_t max_query_len, int32_t num_tokens,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                         float scale, bool may_split, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    if (!pool || pool->host) return KV_ERR_INVALID_ARG;
    const kv_pool_desc_t& d = pool->desc;
    if (layer < 0 || layer >= d.num_layers || batch < 0 || max_query_len < 0 || num_q_heads < 1)
        return KV_ERR_INVALID_ARG;
    if (num_q_heads % d.num_kv_heads != 0) return KV_ERR_UNSUPPORTED;
    if (num_q_heads / d.num_kv_heads > pkv::kMaxGroup) return KV_ERR_UNSUPPORTED;
    if (!(scale == scale)) return KV_ERR_INVALID_ARG;
    if (batch == 0 || max_query_len == 0) return KV_OK;
    if (max_blocks_per_seq < 1) return KV_ERR_INVALID_ARG;
    if (!out || !query || !query_start || !block_tables || !context_lens) return KV_ERR_INVALID_ARG;
    if (!aligned(out) || !aligned(query) || !aligned(query_start, 4) || !aligned(block_tables, 4) ||
        !aligned(context_lens, 4))
        return KV_ERR_INVALID_ARG;
    if (static_cast<int64_t>(max_blocks_per_seq) * d.block_size > INT32_MAX) return KV_ERR_INVALID_ARG;
    PrefillPlan pl;
    kv_status_t st = plan_prefill(pool, batch, num_q_heads, max_query_len, max_blocks_per_seq,
                                  may_split, &pl);
    if (st != KV_OK) return st;
    if (pl.row_tiles > INT32_MAX ||
        static_cast<int64_t>(batch) * d.num_kv_heads * pl.row_tiles * pl.splits > INT32_MAX)
        return KV_ERR_INVALID_ARG;
    size_t ml_offset = 0;
    if (pl.splits > 1) {
        if (num_tokens < 1) return KV_ERR_INVALID_ARG;
        if (prefill_partial_bytes(num_tokens, num_q_heads, d.head_dim, pl.splits, &ml_offset) > workspace_bytes)
            return KV_ERR_WORKSPACE;
        if (!workspace || !aligned(workspace, 256)) return KV_ERR_INVALID_ARG;
    }
    if (checked_mode()) {
        st = check_tables_on_device(pool, block_tables, max_blocks_per_seq, context_lens, batch, stream);
        if (st == KV_OK)
            st = run_check(0, stream, [&](uint32_t* status, uint32_t*) {
                return pkv::launch_check_query_start(query_start, batch, max_query_len, status, stream);
            });
        if (st != KV_OK) return st;
    }
    DecodeShape shape;
    shape.group = pl.group;
    shape.part_blocks = 1;
    shape.num_parts = 1;
    pkv::PrefillArgs pa;
    pa.a = make_args(pool, layer, out, query, block_tables, max_blocks_per_seq, context_lens,
                     batch, num_q_heads, scale, nullptr, shape);
    pa.a.stream_loads = 0;       // keys are re-read by every row tile of a sequence
    pa.a.streamed = 0;
    pa.qstart = query_start;
    pa.group = pl.group;
    pa.row_tiles = static_cast<int32_t>(pl.row_tiles);
    pa.waves = pl.waves;
    pa.buffer_bytes = pool->cache_bytes < (size_t(1) << 31) ? static_cast<int32_t>(pool->cache_bytes) : 0;
    pa.splits = pl.splits;
    pa.num_tokens = num_tokens;
    pa.ws_acc = pl.splits > 1 ? static_cast<float*>(workspace) : nullptr;
    pa.ws_ml = pl.splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + ml_offset) : nullptr;
    pa.dense_len = 0;
    return pkv::launch_prefill(d.dtype, io_dtype(d), d.head_dim, pa, stream) == hipSuccess
               ? KV_OK
               : KV_ERR_HIP;
}

// ---- decode over a shared prefix (see paged_attention_decode_shared_prefix)

constexpr int kMaxCascadeSplits = 64;

// The launch shape of a shared-prefix decode (host values only).
struct CascadePlan {
    int32_t group = 0;
    int waves = 4;              // prefix pass: waves per work-group
    int64_t row_tiles = 0;      // prefix pass: row tiles per KV head (batch * group rows)
    int splits = 1;             // prefix pass: work-groups sharing each row tile's keys
    int32_t suffix_blocks = 0;  // table entries after the prefix
    DecodeShape suffix;         // the suffix's partition shape (num_parts 0 if no entries)
    size_t pre_ml_offset = 0;   // prefix partials: int16 acc at 0, (m, l, scale, 0) here
    size_t suffix_offset = 0;   // suffix partials (acc, then (m, l)) from here
    size_t total = 0;           // workspace bytes
    bool fused = false;         // every suffix in one partition: the suffix kernel combines
                                // the prefix partials and writes the output (no reduce)
};

// Suffixes up to this many tokens (the table width after the prefix) are walked as one
// partition, so that the suffix kernel can write the final output itself.
constexpr int32_t kFusedSuffixTokens = 1024;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// bytes of the prefix pass's partial results: int16 accumulators, then (m, l, scale, 0)
size_t dense_partial_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim, int splits,
                           size_t* ml_offset) {
    const size_t parts = static_cast<size_t>(batch) * num_q_heads * splits;
    const size_t acc = align256(parts * head_dim * sizeof(int16_t));
    if (ml_offset) *ml_offset = acc;
    return acc + parts * 4 * sizeof(float);
}

kv_status_t plan_cascade(const kv_pool_t* pool, int32_t batch, int32_t num_q_heads,
                         int32_t max_blocks, int32_t prefix_blocks, int32_t partition_size,
                         CascadePlan* cp) {
    const kv_pool_desc_t& d = pool->desc;
    if (batch < 1 || num_q_heads < 1 || max_blocks < 1 || prefix_blocks < 1 || prefix_blocks > max_blocks)
        return KV_ERR_INVALID_ARG;
    if (num_q_heads % d.num_kv_heads != 0) return KV_ERR_UNSUPPORTED;
    cp->group = num_q_heads / d.num_kv_heads;
    if (cp->group > pkv::kMaxGroup) return KV_ERR_UNSUPPORTED;
    if (partition_size == 0) partition_size = pkv::kDefaultPartition;
    if (partition_size < d.block_size || partition_size % d.block_size != 0) return KV_ERR_INVALID_ARG;
    if (static_cast<int64_t>(max_blocks) * d.block_size > INT32_MAX) return KV_ERR_INVALID_ARG;
    // prefix pass: the batch's query rows of a KV head are one row range; 8-wave
    // work-groups (256 rows) stage each key once for all of them when there are that many
    // (PAGEDKV_PREFILL_WAVES=4|8 forces the choice)
    const int64_t rows = static_cast<int64_t>(batch) * cp->group;
    const char* ew = getenv("PAGEDKV_PREFILL_WAVES");
    const int forced = ew ? atoi(ew) : 0;
    cp->waves = (forced == 4 || forced == 8) ? forced : (rows >= 256 ? 8 : 4);
    cp->row_tiles = ceil_div(rows, 32 * cp->waves);
    const int64_t wgs = static_cast<int64_t>(d.num_kv_heads) * cp->row_tiles;
    int64_t resident = pkv::prefill_resident_groups(d.dtype, io_dtype(d), d.head_dim, cp->waves);
    if (resident <= 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
            (void)hipGetLastError();
            cus = 256;
        }
        resident = 2 * static_cast<int64_t>(cus);     // no occupancy known: two per CU
    }
    // enough work-groups to fill the resident slots, each with at least two 64-key stages
    const int64_t stages = ceil_div(static_cast<int64_t>(prefix_blocks) * d.block_size, 64);
    int64_t splits = wgs < resident ? ceil_div(resident, wgs) : 1;
    splits = std::min<int64_t>({splits, kMaxCascadeSplits, std::max<int64_t>(1, stages / 2)});
    const char* e = getenv("PAGEDKV_CASCADE_SPLITS");
    if (e && atoi(e) >= 1) splits = std::min(atoi(e), kMaxCascadeSplits);
    cp->splits = static_cast<int>(splits);
    if (wgs * cp->splits > INT32_MAX) return KV_ERR_INVALID_ARG;
    const size_t pre = dense_partial_bytes(batch, num_q_heads, d.head_dim, cp->splits, &cp->pre_ml_offset);
    // suffix pass: the decode's shape over the entries after the prefix; its partial
    // results are kept even for a single partition
    cp->suffix_blocks = max_blocks - prefix_blocks;
    cp->suffix = DecodeShape();
    cp->suffix.group = cp->group;
    cp->suffix_offset = align256(pre);
    cp->total = cp->suffix_offset;
    if (cp->suffix_blocks > 0) {
        const int32_t tile = d.block_size < pkv::kTile ? d.block_size : pkv::kTile;
        if (partition_size > pkv::kMaxPartition || partition_size > pkv::kMaxTilesPerWave * tile)
            return KV_ERR_UNSUPPORTED;
        // one partition per suffix when the table width after the prefix allows it
        // (PAGEDKV_CASCADE_FUSE=0: partial results and the cascade reduce instead)
        const int64_t width = static_cast<int64_t>(cp->suffix_blocks) * d.block_size;
        const char* ef = getenv("PAGEDKV_CASCADE_FUSE");
        if (!(ef && ef[0] == '0') && width <= std::max<int64_t>(partition_size, kFusedSuffixTokens)) {
            cp->fused = true;
            cp->suffix.part_blocks = static_cast<int32_t>(std::max<int64_t>(width, partition_size) / tile);
            cp->suffix.num_parts = 1;
            cp->suffix.ws_needed = 0;
            return KV_OK;
        }
        cp->suffix.part_blocks = partition_size / tile;
        cp->suffix.num_parts = static_cast<int32_t>(
            ceil_div(static_cast<int64_t>(cp->suffix_blocks) * d.block_size, partition_size));
        if (static_cast<int64_t>(batch) * d.num_kv_heads * cp->suffix.num_parts > INT32_MAX)
            return KV_ERR_INVALID_ARG;
        const size_t n = static_cast<size_t>(batch) * num_q_heads * cp->suffix.num_parts;
        cp->suffix.ws_needed = align256(n * d.head_dim * sizeof(float)) + n * 2 * sizeof(float);
        cp->total += cp->suffix.ws_needed;
    }
    return KV_OK;
}

kv_status_t shared_prefix_impl(const kv_pool_t* pool, int32_t layer, void* out, const void* query,
                               const void* new_key, const void* new_value,
                               const int32_t* block_tables, int32_t max_blocks,
                               const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                               float scale, int32_t prefix_blocks, int32_t partition_size,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if ((new_key == nullptr) != (new_value == nullptr)) return KV_ERR_INVALID_ARG;
    if (new_key && (!aligned(new_key) || !aligned(new_value))) return KV_ERR_INVALID_ARG;
    if (prefix_blocks == 0)
        return decode_impl(kBoth, pool, layer, out, query, block_tables, max_blocks, context_lens,
                           batch, num_q_heads, scale, partition_size, workspace, workspace_bytes,
                           stream, new_key, new_value);
    DecodeShape s;
    kv_status_t st = check_decode(pool, layer, out, query, block_tables, max_blocks, context_lens,
                                  batch, num_q_heads, scale, partition_size, nullptr, 0, &s, false);
    if (st != KV_OK) return st;
    if (prefix_blocks < 0 || (batch > 0 && prefix_blocks > max_blocks)) return KV_ERR_INVALID_ARG;
    if (batch == 0) return KV_OK;
    // a new token at position L - 1 needs a table entry after the prefix
    if (new_key && prefix_blocks == max_blocks) return KV_ERR_INVALID_ARG;
    CascadePlan cp;
    st = plan_cascade(pool, batch, num_q_heads, max_blocks, prefix_blocks, partition_size, &cp);
    if (st != KV_OK) return st;
    if (!workspace || workspace_bytes < cp.total) return KV_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return KV_ERR_INVALID_ARG;
    const kv_pool_desc_t& d = pool->desc;
    if (checked_mode()) {
        st = check_tables_on_device(pool, block_tables, max_blocks, context_lens, batch, stream);
        if (st == KV_OK)
            st = run_check(0, stream, [&](uint32_t* status, uint32_t*) {
                return pkv::launch_check_shared_prefix(block_tables, max_blocks, context_lens, batch,
                                                       prefix_blocks, d.block_size, new_key ? 1 : 0,
                                                       status, stream);
            });
        if (st == KV_OK && new_key) {
            const int64_t slots = static_cast<int64_t>(d.num_blocks) * d.block_size;
            st = run_check(slots, stream, [&](uint32_t* status, uint32_t* seen) {
                return pkv::launch_check_append_slots(block_tables, max_blocks, context_lens, batch,
                                                      d.num_blocks, d.block_size, seen, status, stream);
            });
        }
        if (st != KV_OK) return st;
    }
    char* ws = static_cast<char*>(workspace);
    const int32_t prefix_len = prefix_blocks * d.block_size;

    // 1. the prefix: every query row against keys [0, prefix_len) of table row 0
    DecodeShape one;
    one.group = cp.group;
    one.part_blocks = 1;
    one.num_parts = 1;
    pkv::PrefillArgs pa;
    pa.a = make_args(pool, layer, out, query, block_tables, max_blocks, context_lens, batch,
                     num_q_heads, scale, nullptr, one);
    pa.a.stream_loads = 0;
    pa.a.streamed = 0;
    pa.qstart = nullptr;
    pa.group = cp.group;
    pa.row_tiles = static_cast<int32_t>(cp.row_tiles);
    pa.waves = cp.waves;
    pa.buffer_bytes = pool->cache_bytes < (size_t(1) << 31) ? static_cast<int32_t>(pool->cache_bytes) : 0;
    pa.splits = cp.splits;
    pa.num_tokens = batch;
    pa.ws_acc = reinterpret_cast<float*>(ws);
    pa.ws_ml = reinterpret_cast<float*>(ws + cp.pre_ml_offset);
    pa.dense_len = prefix_len;
    if (pkv::launch_prefill_dense(d.dtype, io_dtype(d), d.head_dim, pa, stream) != hipSuccess)
        return KV_ERR_HIP;

    // 2. the suffixes: the decode over the entries after the prefix, partial results kept
    //    (fused: one partition per suffix, combined with the prefix's partials and written
    //    as the output by the suffix kernel itself; a sequence without a suffix too)
    pkv::DecodeArgs a = make_args(pool, layer, out, query, block_tables + prefix_blocks,
                                  cp.suffix_blocks, context_lens, batch, num_q_heads, scale,
                                  ws + cp.suffix_offset, cp.suffix);
    a.table_stride = max_blocks;
    a.len_offset = prefix_len;
    if (cp.fused) {
        a.pre_acc = reinterpret_cast<const int16_t*>(pa.ws_acc);
        a.pre_ml = pa.ws_ml;
        a.pre_parts = cp.splits;
        a.new_k = static_cast<const uint16_t*>(new_key);
        a.new_v = static_cast<const uint16_t*>(new_value);
        return pkv::launch_partitions(d.dtype, io_dtype(d), d.head_dim, cp.group, a, stream) == hipSuccess
                   ? KV_OK
                   : KV_ERR_HIP;
    }
    a.keep_partials = 1;
    pkv::DecodeArgs r = a;
    if (cp.suffix_blocks > 0) {
        a.new_k = static_cast<const uint16_t*>(new_key);
        a.new_v = static_cast<const uint16_t*>(new_value);
        if (pkv::launch_partitions(d.dtype, io_dtype(d), d.head_dim, cp.group, a, stream) != hipSuccess)
            return KV_ERR_HIP;
        const int chunk = pkv::partition_chunk(d.dtype, io_dtype(d), d.head_dim, cp.group, a);
        r.part_blocks = a.part_blocks * chunk;
        r.num_parts = static_cast<int32_t>(ceil_div(a.num_parts, chunk));
    } else {
        r.part_blocks = 1;      // no entries: every suffix is empty
        r.num_parts = 1;
    }

    // 3. prefix and suffix partial results combined per (sequence, query head)
    return pkv::launch_cascade_reduce(io_dtype(d), d.head_dim, r,
                                      reinterpret_cast<const int16_t*>(pa.ws_acc), pa.ws_ml,
                                      cp.splits, stream) == hipSuccess
               ? KV_OK
               : KV_ERR_HIP;
}

}  // namespace

extern "C" {

const char* kv_status_string(kv_status_t status) {
    switch (status) {
        case KV_OK: return "ok";
        case KV_ERR_INVALID_ARG: return "invalid argument";
        case KV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case KV_ERR_WORKSPACE: return "workspace missing or too small";
        case KV_ERR_OUT_OF_MEMORY: return "out of device memory";
        case KV_ERR_HIP: return "HIP runtime error";
        case KV_ERR_OUT_OF_BLOCKS: return "no free block";
    }
    return "unknown status";
}

size_t kv_bytes_per_token(const kv_pool_desc_t* desc) {
    if (check_desc(desc) != KV_OK) return 0;
    return 2u * static_cast<size_t>(desc->num_layers) * desc->num_kv_heads * desc->head_dim *
           elem_bytes(*desc);
}

size_t kv_pool_bytes(const kv_pool_desc_t* desc) {
    if (check_desc(desc) != KV_OK) return 0;
    return kv_bytes_per_token(desc) * static_cast<size_t>(desc->num_blocks) * desc->block_size;
}

kv_status_t kv_pool_create(const kv_pool_desc_t* desc, void* device_base, size_t base_bytes,
                           kv_pool_t** out) {
    if (!out) return KV_ERR_INVALID_ARG;
    const kv_status_t st = check_desc(desc);
    if (st != KV_OK) return st;
    const size_t need = kv_pool_bytes(desc);
    if (device_base) {
        if (!aligned(device_base, 256) || base_bytes < need) return KV_ERR_INVALID_ARG;
    }
    kv_pool_t* p = new (std::nothrow) kv_pool_t;
    if (!p) return KV_ERR_OUT_OF_MEMORY;
    p->desc = *desc;
    p->cache_bytes = cache_bytes(desc);
    p->owned = 0;
    p->host = 0;
    p->host_base = nullptr;
    p->device = -1;
    if (hipGetDevice(&p->device) != hipSuccess) {
        (void)hipGetLastError();
        p->device = -1;
        if (!device_base) {      // allocation needs a device
            delete p;
            return KV_ERR_HIP;
        }
    }
    if (device_base) {
        p->base = static_cast<char*>(device_base);
    } else {
        void* mem = nullptr;
        if (hipMalloc(&mem, need) != hipSuccess || !mem) {
            (void)hipGetLastError();
            delete p;
            return KV_ERR_OUT_OF_MEMORY;
        }
        p->base = static_cast<char*>(mem);
        p->owned = 1;
    }
    *out = p;
    return KV_OK;
}

kv_status_t kv_host_pool_create(const kv_pool_desc_t* desc, void* host_base, size_t base_bytes,
                                kv_pool_t** out) {
    if (!out) return KV_ERR_INVALID_ARG;
    const kv_status_t st = check_desc(desc);
    if (st != KV_OK) return st;
    const size_t need = kv_pool_bytes(desc);
    if (host_base && (!aligned(host_base, 256) || base_bytes < need)) return KV_ERR_INVALID_ARG;
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess) {
        (void)hipGetLastError();
        return KV_ERR_HIP;
    }
    void* host = host_base;
    int owned = 0;
    if (!host) {
        if (hipHostMalloc(&host, need, hipHostMallocDefault) != hipSuccess || !host) {
            (void)hipGetLastError();
            return KV_ERR_OUT_OF_MEMORY;
        }
        owned = 1;
    } else {
        // the kernels reach the memory through its device mapping: it must be pinned
        // host memory HIP knows, and both ends of the range must map
        hipPointerAttribute_t attr;
        if (hipPointerGetAttributes(&attr, host_base) != hipSuccess ||
            attr.type != hipMemoryTypeHost) {
            (void)hipGetLastError();
            return KV_ERR_INVALID_ARG;
        }
        void* last = nullptr;
        if (hipHostGetDevicePointer(&last, static_cast<char*>(host_base) + need - 1, 0) !=
                hipSuccess || !last) {
            (void)hipGetLastError();
            return KV_ERR_INVALID_ARG;
        }
    }
    void* dev = nullptr;
    if (hipHostGetDevicePointer(&dev, host, 0) != hipSuccess || !dev) {
        (void)hipGetLastError();
        if (owned) (void)hipHostFree(host);
        return KV_ERR_INVALID_ARG;
    }
    kv_pool_t* p = new (std::nothrow) kv_pool_t;
    if (!p) {
        if (owned) (void)hipHostFree(host);
        return KV_ERR_OUT_OF_MEMORY;
    }
    p->desc = *desc;
    p->cache_bytes = cache_bytes(desc);
    p->owned = owned;
    p->host = 1;
    p->host_base = static_cast<char*>(host);
    p->base = static_cast<char*>(dev);
    p->device = device;
    *out = p;
    return KV_OK;
}

int32_t kv_pool_is_host(const kv_pool_t* pool) { return pool ? pool->host : -1; }

kv_status_t kv_pool_destroy(kv_pool_t* pool) {
    if (!pool) return KV_OK;
    kv_status_t st = KV_OK;
    if (pool->owned) {
        const hipError_t e = pool->host ? hipHostFree(pool->host_base) : hipFree(pool->base);
        if (e != hipSuccess) st = KV_ERR_HIP;
    }
    delete pool;
    return st;
}

kv_status_t kv_pool_get_desc(const kv_pool_t* pool, kv_pool_desc_t* desc) {
    if (!pool || !desc) return KV_ERR_INVALID_ARG;
    *desc = pool->desc;
    return KV_OK;
}

kv_status_t kv_pool_layer_ptrs(const kv_pool_t* pool, int32_t layer, void** k_cache,
                               void** v_cache) {
    if (!pool || layer < 0 || layer >= pool->desc.num_layers) return KV_ERR_INVALID_ARG;
    char* kc = (pool->host ? pool->host_base : pool->base) +
               static_cast<size_t>(2 * layer) * pool->cache_bytes;
    if (k_cache) *k_cache = kc;
    if (v_cache) *v_cache = kc + pool->cache_bytes;
    return KV_OK;
}

kv_status_t reshape_and_cache(kv_pool_t* pool, int32_t layer, const void* key, const void* value,
                              const int64_t* slot_mapping, int32_t num_tokens, hipStream_t stream) {
    if (!pool || pool->host || layer < 0 || layer >= pool->desc.num_layers || num_tokens < 0)
        return KV_ERR_INVALID_ARG;
    if (num_tokens == 0) return KV_OK;
    if (!key || !value || !slot_mapping) return KV_ERR_INVALID_ARG;
    if (!aligned(key) || !aligned(value) || !aligned(slot_mapping, 8)) return KV_ERR_INVALID_ARG;
    const kv_pool_desc_t& d = pool->desc;
    char* kc = pool->base + static_cast<size_t>(2 * layer) * pool->cache_bytes;
    const int64_t num_slots = static_cast<int64_t>(d.num_blocks) * d.block_size;
    if (checked_mode()) {
        const kv_status_t st = run_check(num_slots, stream, [&](uint32_t* status, uint32_t* seen) {
            return pkv::launch_check_slots(slot_mapping, num_tokens, num_slots, seen, status, stream);
        });
        if (st != KV_OK) return st;
    }
    const hipError_t e = pkv::launch_reshape_and_cache(
        key, value, slot_mapping, num_tokens, kc, kc + pool->cache_bytes, num_slots,
        d.num_kv_heads * d.head_dim, d.dtype, io_dtype(d), stream);
    return e == hipSuccess ? KV_OK : KV_ERR_HIP;
}

kv_status_t kv_copy_blocks(kv_pool_t* pool, const int32_t* copies, int32_t num_copies,
                           hipStream_t stream) {
    if (!pool || pool->host || num_copies < 0) return KV_ERR_INVALID_ARG;
    if (num_copies == 0) return KV_OK;
    if (!copies || !aligned(copies, 4)) return KV_ERR_INVALID_ARG;
    const kv_pool_desc_t& d = pool->desc;
    const hipError_t e = pkv::launch_copy_blocks(
        pool->base, copies, num_copies, d.num_layers, d.num_blocks, d.block_size,
        d.num_kv_heads * d.head_dim * static_cast<int32_t>(elem_bytes(d)), pool->cache_bytes,
        stream);
    return e == hipSuccess ? KV_OK : KV_ERR_HIP;
}

kv_status_t kv_swap_blocks(const kv_pool_t* src, kv_pool_t* dst, const int32_t* pairs,
                           int32_t num_pairs, hipStream_t stream) {
    if (!src || !dst || src == dst || num_pairs < 0) return KV_ERR_INVALID_ARG;
    const kv_pool_desc_t& a = src->desc;
    const kv_pool_desc_t& b = dst->desc;
    if (a.num_layers != b.num_layers || a.block_size != b.block_size ||
        a.num_kv_heads != b.num_kv_heads || a.head_dim != b.head_dim || a.dtype != b.dtype)
        return KV_ERR_INVALID_ARG;
    if (num_pairs == 0) return KV_OK;
    if (!pairs || !aligned(pairs, 8)) return KV_ERR_INVALID_ARG;
    const size_t block_bytes = static_cast<size_t>(a.block_size) * a.num_kv_heads * a.head_dim *
                               elem_bytes(a);
    const hipError_t e = pkv::launch_swap_blocks(src->base, dst->base, pairs, num_pairs,
                                                 a.num_layers, a.num_blocks, b.num_blocks,
                                                 block_bytes, src->cache_bytes, dst->cache_bytes,
                                                 stream);
    return e == hipSuccess ? KV_OK : KV_ERR_HIP;
}

size_t paged_attention_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                       int32_t max_blocks_per_seq, int32_t block_size,
                                       int32_t partition_size) {
    if (batch < 0 || num_q_heads < 1 || head_dim < 1 || max_blocks_per_seq < 1 ||
        (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64))
        return SIZE_MAX;
    if (partition_size == 0) partition_size = pkv::kDefaultPartition;
    if (partition_size < block_size || partition_size % block_size != 0) return SIZE_MAX;
    const int32_t parts = static_cast<int32_t>(
        ceil_div(static_cast<int64_t>(max_blocks_per_seq) * block_size, partition_size));
    return workspace_for(batch, num_q_heads, head_dim, parts);
}

kv_status_t paged_attention_decode(const kv_pool_t* pool, int32_t layer, void* out,
                                   const void* query, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* context_lens,
                                   int32_t batch, int32_t num_q_heads, float scale,
                                   int32_t partition_size, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    return decode_impl(kBoth, pool, layer, out, query, block_tables, max_blocks_per_seq,
                       context_lens, batch, num_q_heads, scale, partition_size, workspace,
                       workspace_bytes, stream);
}

kv_status_t paged_attention_partitions(const kv_pool_t* pool, int32_t layer, void* out,
                                       const void* query, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                                       int32_t batch, int32_t num_q_heads, float scale,
                                       int32_t partition_size, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    return decode_impl(kPartitions, pool, layer, out, query, block_tables, max_blocks_per_seq,
                       context_lens, batch, num_q_heads, scale, partition_size, workspace,
                       workspace_bytes, stream);
}

kv_status_t paged_attention_prefill(const kv_pool_t* pool, int32_t layer, void* out,
                                    const void* query, const int32_t* query_start,
                                    int32_t max_query_len, const int32_t* block_tables,
                                    int32_t max_blocks_per_seq, const int32_t* context_lens,
                                    int32_t batch, int32_t num_q_heads, float scale,
                                    hipStream_t stream) {
    return prefill_impl(pool, layer, out, query, query_start, max_query_len, 0, block_tables,
                        max_blocks_per_seq, context_lens, batch, num_q_heads, scale, false,
                        nullptr, 0, stream);
}

size_t paged_attention_prefill_workspace_bytes(const kv_pool_t* pool, int32_t batch,
                                               int32_t num_q_heads, int32_t num_tokens,
                                               int32_t max_query_len, int32_t max_blocks_per_seq) {
    if (!pool || batch < 1 || num_q_heads < 1 || num_tokens < 1 || max_query_len < 1 ||
        max_blocks_per_seq < 1)
        return 0;
    PrefillPlan pl;
    if (plan_prefill(pool, batch, num_q_heads, max_query_len, max_blocks_per_seq, true, &pl) != KV_OK ||
        pl.splits <= 1)
        return 0;
    return prefill_partial_bytes(num_tokens, num_q_heads, pool->desc.head_dim, pl.splits, nullptr);
}

kv_status_t paged_attention_prefill_split(const kv_pool_t* pool, int32_t layer, void* out,
                                          const void* query, const int32_t* query_start,
                                          int32_t max_query_len, int32_t num_tokens,
                                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t batch,
                                          int32_t num_q_heads, float scale, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
    return prefill_impl(pool, layer, out, query, query_start, max_query_len, num_tokens,
                        block_tables, max_blocks_per_seq, context_lens, batch, num_q_heads, scale,
                        true, workspace, workspace_bytes, stream);
}

kv_status_t paged_attention_decode_append(const kv_pool_t* pool, int32_t layer, void* out,
                                          const void* query, const void* new_key,
                                          const void* new_value, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                                          int32_t batch, int32_t num_q_heads, float scale,
                                          int32_t partition_size, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
    if (batch > 0 && (!new_key || !new_value || !aligned(new_key) || !aligned(new_value)))
        return KV_ERR_INVALID_ARG;
    return decode_impl(kBoth, pool, layer, out, query, block_tables, max_blocks_per_seq,
                       context_lens, batch, num_q_heads, scale, partition_size, workspace,
                       workspace_bytes, stream, new_key, new_value);
}

kv_status_t paged_attention_partitions_append(const kv_pool_t* pool, int32_t layer, void* out,
                                              const void* query, const void* new_key,
                                              const void* new_value, const int32_t* block_tables,
                                              int32_t max_blocks_per_seq,
                                              const int32_t* context_lens, int32_t batch,
                                              int32_t num_q_heads, float scale,
                                              int32_t partition_size, void* workspace,
                                              size_t workspace_bytes, hipStream_t stream) {
    if (batch > 0 && (!new_key || !new_value || !aligned(new_key) || !aligned(new_value)))
        return KV_ERR_INVALID_ARG;
    return decode_impl(kPartitions, pool, layer, out, query, block_tables, max_blocks_per_seq,
                       context_lens, batch, num_q_heads, scale, partition_size, workspace,
                       workspace_bytes, stream, new_key, new_value);
}

kv_status_t paged_attention_reduce(const kv_pool_t* pool, int32_t layer, void* out,
                                   const void* query, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* context_lens,
                                   int32_t batch, int32_t num_q_heads, float scale,
                                   int32_t partition_size, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    return decode_impl(kReduce, pool, layer, out, query, block_tables, max_blocks_per_seq,
                       context_lens, batch, num_q_heads, scale, partition_size, workspace,
                       workspace_bytes, stream);
}

kv_status_t paged_attention_decode_noalloc(const kv_pool_t* pool, int32_t layer, void* out,
                                           const void* query, const int32_t* block_tables,
                                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                                           int32_t batch, int32_t num_q_heads, float scale,
                                           int32_t partition_size, hipStream_t stream) {
    if (!pool || pool->host) return KV_ERR_INVALID_ARG;
    // SIZE_MAX: arguments the decode checks below refuse
    const size_t need = batch > 0 ? paged_attention_workspace_bytes(batch, num_q_heads,
                                                                    pool->desc.head_dim,
                                                                    max_blocks_per_seq,
                                                                    pool->desc.block_size,
                                                                    partition_size)
                                  : 0;
    if (need != SIZE_MAX && need > PAGEDKV_SCRATCH_BYTES) return KV_ERR_WORKSPACE;
    void* scratch = nullptr;
    if (need > 0 && need != SIZE_MAX && pkv::scratch_for_current_device(&scratch) != hipSuccess) {
        (void)hipGetLastError();
        return KV_ERR_HIP;
    }
    // the checked-mode passes allocate and synchronise: not on this path
    return decode_impl(kBoth, pool, layer, out, query, block_tables, max_blocks_per_seq,
                       context_lens, batch, num_q_heads, scale, partition_size, scratch,
                       scratch ? PAGEDKV_SCRATCH_BYTES : 0, stream, nullptr, nullptr, false);
}

kv_status_t kv_pool_gather(const kv_pool_t* pool, int32_t layer, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t batch, void* k_out, void* v_out, hipStream_t stream) {
    if (!pool || pool->host || layer < 0 || layer >= pool->desc.num_layers || batch < 0)
        return KV_ERR_INVALID_ARG;
    if (batch == 0) return KV_OK;
    if (max_blocks_per_seq < 1 || batch > 65535 ||
        max_blocks_per_seq > 0x7fffffff / pool->desc.block_size)
        return KV_ERR_INVALID_ARG;
    if (!block_tables || !context_lens || !k_out || !v_out) return KV_ERR_INVALID_ARG;
    if (!aligned(k_out) || !aligned(v_out) || !aligned(block_tables, 4) || !aligned(context_lens, 4))
        return KV_ERR_INVALID_ARG;
    const kv_pool_desc_t& d = pool->desc;
    const char* kc = pool->base + static_cast<size_t>(2 * layer) * pool->cache_bytes;
    const hipError_t e = pkv::launch_gather(
        kc, kc + pool->cache_bytes, block_tables, max_blocks_per_seq, context_lens, batch,
        d.num_blocks, d.block_size, d.num_kv_heads * d.head_dim * static_cast<int32_t>(elem_bytes(d)),
        k_out, v_out, stream);
    return e == hipSuccess ? KV_OK : KV_ERR_HIP;
}

size_t paged_attention_shared_prefix_workspace_bytes(const kv_pool_t* pool, int32_t batch,
                                                     int32_t num_q_heads, int32_t max_blocks_per_seq,
                                                     int32_t prefix_blocks, int32_t partition_size) {
    if (!pool || pool->host || batch < 0 || num_q_heads < 1 || max_blocks_per_seq < 1 ||
        prefix_blocks < 0 || prefix_blocks > max_blocks_per_seq)
        return SIZE_MAX;
    if (prefix_blocks == 0 || batch == 0)
        return batch == 0 ? 0
                          : paged_attention_workspace_bytes(batch, num_q_heads, pool->desc.head_dim,
                                                            max_blocks_per_seq, pool->desc.block_size,
                                                            partition_size);
    CascadePlan cp;
    if (plan_cascade(pool, batch, num_q_heads, max_blocks_per_seq, prefix_blocks, partition_size, &cp) != KV_OK)
        return SIZE_MAX;
    return cp.total;
}

kv_status_t paged_attention_decode_shared_prefix(const kv_pool_t* pool, int32_t layer, void* out,
                                                 const void* query, const void* new_key,
                                                 const void* new_value, const int32_t* block_tables,
                                                 int32_t max_blocks_per_seq,
                                                 const int32_t* context_lens, int32_t batch,
                                                 int32_t num_q_heads, float scale,
                                                 int32_t prefix_blocks, int32_t partition_size,
                                                 void* workspace, size_t workspace_bytes,
                                                 hipStream_t stream) {
    return shared_prefix_impl(pool, layer, out, query, new_key, new_value, block_tables,
                              max_blocks_per_seq, context_lens, batch, num_q_heads, scale,
                              prefix_blocks, partition_size, workspace, workspace_bytes, stream);
}

}  // extern "C"
