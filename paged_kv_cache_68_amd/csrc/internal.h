// Internal declarations shared by the C ABI (api.cpp) and the HIP kernel files.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "pagedkv.h"

struct kv_pool {
    kv_pool_desc_t desc;
    char* base;          // device address of layer 0's K cache (device view of a host pool)
    char* host_base;     // host address of a host pool, else nullptr
    int owned;           // 1 if the library allocated the memory
    int host;            // 1 for a pool in pinned host memory
    int device;          // HIP device the pool lives on (mapped for, if host)
    size_t cache_bytes;  // bytes of one layer's K (or V) cache
};

namespace pkv {

constexpr int kBlockSize = 16;          // default tokens per physical block (the VALU kernel's)
constexpr int kTile = 16;               // tokens per matrix-core tile
constexpr int kDefaultSwapGroups = 64;  // work-groups of a swap copy (host-link bound)
constexpr int kMaxTilesPerWave = 256;   // a wave holds one table entry per tile in 4 VGPRs
constexpr int kDefaultPartition = 512;  // tokens per split-context partition
constexpr int kMaxPartition = 4096;     // at most 256 tiles of 16 tokens per wave
constexpr int kMaxGroup = 16;           // largest supported GQA group (MFMA path)
constexpr int kMaxGroupValu = 8;        // largest group the VALU kernel is built for
constexpr int kWavesPerGroup = 4;       // waves per work-group of the partition kernel

// Everything the two decode kernels read; passed by value.
struct DecodeArgs {
    const uint16_t* q;       // [B][Hq][D]
    const uint8_t* k;        // [nb][block_size][Hkv][D], elements of the storage type
    const uint8_t* v;
    int32_t row_bytes;       // bytes of one token row of K (Hkv * D * element bytes)
    const int32_t* tables;   // [B][table_stride], max_blocks entries of each row used
    const int32_t* lens;     // [B]: context lengths; the kernels see lens[b] - len_offset
    uint16_t* out;           // [B][Hq][D]
    const uint16_t* new_k;   // [B][Hkv][D] io type, or null: the token at position L - 1 of
    const uint16_t* new_v;   // each sequence, written into its slot (found through the
                             // table) before it is read, in the same launch
    float* ws_acc;           // [B][Hkv][P][G][D]  unnormalised accumulators
    float* ws_ml;            // [B][Hkv][P][G][2]  (running max in log2 units, running sum)
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t max_blocks;      // table entries per sequence (from `tables` on)
    int32_t table_stride;    // entries between two sequences' rows (>= max_blocks)
    int32_t len_offset;      // tokens before the table's first entry (a shared prefix
                             // handled elsewhere): a sequence holds lens[b] - len_offset
    int32_t keep_partials;   // 1: every sequence's partitions go to the workspace as
                             // partial results, even a single one (no final output is
                             // written; a sequence without tokens writes nothing)
    const int16_t* pre_acc;  // pre_parts > 0: a shared prefix's partial results, combined
    const float* pre_ml;     // with each sequence's (single-partition) result before it is
    int32_t pre_parts;       // written: [B][Hq][pre_parts][D] int16 accumulators and
                             // [B][Hq][pre_parts] (m, l, scale, 0)
    int32_t num_blocks;      // blocks in the pool
    int32_t block_size;      // tokens per block: 8, 16, 32 or 64
    int32_t tile_tokens;     // tokens per tile the kernels walk: min(block_size, 16)
    int32_t tiles_log2;      // log2(block_size / tile_tokens): tiles per block
    int32_t part_blocks;     // tiles per partition (tiles are blocks when block_size <= 16)
    int32_t num_parts;       // partitions of the longest possible sequence
    float scale_log2;        // scale * log2(e): scores are kept in base-2 units
    int32_t xcd_chunk;       // work-groups per XCD chunk in the launch renumbering
    int32_t stream_loads;    // 1: K/V loads carry the non-temporal hint
    int32_t streamed;        // 1: the call reaches more K/V bytes than the last-level
                             // cache holds (the plan's input; the hint can be overridden)
    int32_t layer_bytes;     // bytes of this layer's K (and V) cache if at most 0x7FF00000,
                             // else 0: lets a wave address any block with 32-bit offsets
    const int32_t* order;    // [B] or null: the group plan's work-groups take sequences in
                             // this order (longest first) instead of batch order
};

// Multi-token (prefill) attention: the decode arguments (queries and outputs are
// [T][Hq][D], packed over the batch) plus where each sequence's queries start.
struct PrefillArgs {
    DecodeArgs a;
    const int32_t* qstart;   // [B + 1]: sequence b's queries are rows [qstart[b], qstart[b+1])
    int32_t group;           // query heads per KV head
    int32_t row_tiles;       // work-groups per (sequence, KV head)
    int32_t waves;           // waves per work-group (4 or 8); 32 rows each
    int32_t buffer_bytes;    // > 0: one layer's K (and V) cache spans this many bytes, small
                             // enough for 32-bit buffer offsets; 0: 64-bit addresses
    int32_t splits;          // work-groups sharing each row tile's key range (1: none)
    int32_t num_tokens;      // (splits > 1) rows of the query: bounds the partial results
    float* ws_acc;           // (splits > 1) [num_tokens * num_q_heads][splits][D]
                             // (dense launch: int16 [..][splits][D], see dense_len)
    float* ws_ml;            // (splits > 1) [num_tokens * num_q_heads][splits][2]: (m, l)
                             // (dense launch: [..][splits][4]: (m, l, scale, 0))
    int32_t dense_len;       // (dense launch) keys [0, dense_len) of table row 0, shared by
                             // the num_tokens queries of a decode batch ([B][Hq][D]):
                             // query t sees the first min(lens[t], dense_len) of them;
                             // each (row, split) leaves acc / scale as int16 and
                             // (m, l, scale)
};

// A call that can touch more K/V bytes than this streams them past the last-level cache
// (256 MB Infinity Cache on MI355X): they could not stay cached until the next step
// anyway.  Smaller working sets (a few sequences, a shared prefix, a small pool) keep
// the default cache policy so that re-reads hit.
constexpr size_t kStreamThresholdBytes = size_t(512) << 20;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// kv_dtype: storage of K and V (KV_DTYPE_*); io_dtype: queries and outputs (16-bit).
hipError_t launch_partitions(int kv_dtype, int io_dtype, int head_dim, int group,
                             const DecodeArgs& a, hipStream_t stream);
hipError_t launch_partitions_mfma(int kv_dtype, int io_dtype, int head_dim, int group,
                                  const DecodeArgs& a, hipStream_t stream);
// Partitions the partition kernel merges by itself before writing partial results
// (the reduce kernel then combines chunks of that many partitions).
int partition_chunk(int kv_dtype, int io_dtype, int head_dim, int group, const DecodeArgs& a);
int partition_chunk_mfma(int kv_dtype, int io_dtype, int group, int head_dim, const DecodeArgs& a);
// Waves per work-group of the matrix-core kernel's group plan for this batch (0: not used).
int group_waves_mfma(int kv_dtype, int io_dtype, int group, int head_dim, const DecodeArgs& a);
hipError_t launch_reduce(int io_dtype, int head_dim, const DecodeArgs& a, hipStream_t stream);
// (token, head) rows one prefill work-group covers.
// waves per work-group for a prefill launch of `seq_heads` (sequence, KV head) pairs of
// up to `rows` rows each
int prefill_waves_for(int64_t seq_heads, int64_t rows);
hipError_t launch_prefill(int kv_dtype, int io_dtype, int head_dim, const PrefillArgs& pa,
                          hipStream_t stream);
// The shared prefix of a decode batch (PrefillArgs::dense_len): grid num_kv_heads x
// row_tiles x splits, partial results always written (splits >= 1).
hipError_t launch_prefill_dense(int kv_dtype, int io_dtype, int head_dim, const PrefillArgs& pa,
                                hipStream_t stream);
// The cascade reduce: each (sequence, query head) combines `pre_parts` partial results of
// its shared prefix ([B * Hq][pre_parts] rows of pre_acc (int16) / pre_ml (m, l, scale, 0),
// as the dense launch leaves them) with the partial
// results the partition kernel left for its suffix (`a` as for launch_reduce, with
// keep_partials set and len_offset the prefix length), in that order.
hipError_t launch_cascade_reduce(int io_dtype, int head_dim, const DecodeArgs& a,
                                 const int16_t* pre_acc, const float* pre_ml, int pre_parts,
                                 hipStream_t stream);
// work-groups of a prefill launch with `waves` waves each that the GPU holds at once
int64_t prefill_resident_groups(int kv_dtype, int io_dtype, int head_dim, int waves);
constexpr int kMaxPrefillSplits = 8;
// New tokens' rows ([T][row_elems] in io_dtype) into their slots: a bit copy for a
// 16-bit pool, E4M3 rounding for an FP8 pool.
hipError_t launch_reshape_and_cache(const void* key, const void* value, const int64_t* slots,
                                    int32_t num_tokens, void* k_cache, void* v_cache,
                                    int64_t num_slots, int32_t row_elems, int kv_dtype,
                                    int io_dtype, hipStream_t stream);
// base: layer 0's K cache; the 2 * num_layers caches follow each other, cache_bytes
// apart; rows of row_bytes bytes.
// checked mode (PAGEDKV_CHECK=1): validation pre-passes, each or-ing bits into *status
hipError_t launch_check_tables(const int32_t* tables, int32_t max_blocks, const int32_t* lens,
                               int32_t batch, int32_t num_blocks, int32_t block_size,
                               uint32_t* status, hipStream_t stream);
hipError_t launch_check_slots(const int64_t* slots, int32_t n, int64_t num_slots, uint32_t* seen,
                              uint32_t* status, hipStream_t stream);
// (decode with the cache write folded in) the slots of position L - 1 are distinct
hipError_t launch_check_append_slots(const int32_t* tables, int32_t max_blocks, const int32_t* lens,
                                     int32_t batch, int32_t num_blocks, int32_t block_size,
                                     uint32_t* seen, uint32_t* status, hipStream_t stream);
// (decode over a shared prefix) used prefix entries equal row 0's; with `appending`, no
// sequence's last position lies in the prefix
hipError_t launch_check_shared_prefix(const int32_t* tables, int32_t max_blocks, const int32_t* lens,
                                      int32_t batch, int32_t prefix_blocks, int32_t block_size,
                                      int32_t appending, uint32_t* status, hipStream_t stream);
hipError_t launch_check_query_start(const int32_t* qs, int32_t batch, int32_t max_query_len,
                                    uint32_t* status, hipStream_t stream);
hipError_t launch_clear_word(uint32_t* w, hipStream_t stream);

hipError_t launch_swap_blocks(const char* src, char* dst, const int32_t* pairs, int32_t num_pairs,
                              int32_t num_layers, int32_t src_blocks, int32_t dst_blocks,
                              size_t block_bytes, size_t src_cache_bytes, size_t dst_cache_bytes,
                              hipStream_t stream);
// the new tokens of a decode step (DecodeArgs::new_k / new_v) into the slots of position
// L - 1, found through the tables: for kernels that do not write them themselves
hipError_t launch_append_kv(int kv_dtype, int io_dtype, const DecodeArgs& a, hipStream_t stream);
// Bytes of the library's per-device scratch array (paged_attention_decode_noalloc).
constexpr size_t kScratchBytes = PAGEDKV_SCRATCH_BYTES;
// Device address of the current device's scratch array (looked up once per device).
hipError_t scratch_for_current_device(void** ptr);
hipError_t launch_copy_blocks(char* base, const int32_t* copies, int32_t num_copies,
                              int32_t num_layers, int32_t num_blocks, int32_t block_size,
                              int32_t row_bytes, size_t cache_bytes, hipStream_t stream);
hipError_t launch_gather(const void* k_cache, const void* v_cache, const int32_t* tables,
                         int32_t max_blocks, const int32_t* lens, int32_t batch,
                         int32_t num_blocks, int32_t block_size, int32_t row_bytes,
                         void* k_out, void* v_out, hipStream_t stream);

}  // namespace pkv
