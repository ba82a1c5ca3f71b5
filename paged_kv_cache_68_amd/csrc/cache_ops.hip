// Cache write (reshape_and_cache), the copy-on-write block copy and the gather test
// hook, for gfx950.
//
// With the pool laid out [num_blocks][B][Hkv][D], slot = block * B + offset is
// directly the index of a contiguous token row of Hkv*D elements, so the write of
// "Why AI servers waste memory, and how paging fixes it" ("The real implementation":
// the token lands in slot `offset` of block table[-1]) is a row copy to row `slot`,
// a bit copy with 16-byte (dwordx4) accesses; into an FP8 pool each value is rounded to
// E4M3 on the way.  The block copy and the gather are bit copies.

#include <stdlib.h>

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "partition_common.h"

namespace pkv {
namespace {

// One work-group per new token; lanes stride over the 16-byte chunks of the row.
__global__ __launch_bounds__(256) void rc_scatter(const uint4* __restrict__ key,
                                                  const uint4* __restrict__ value,
                                                  const int64_t* __restrict__ slots,
                                                  uint4* __restrict__ k_cache,
                                                  uint4* __restrict__ v_cache, int64_t num_slots,
                                                  int32_t row_chunks) {
    const int64_t i = blockIdx.x;
    const int64_t slot = slots[i];
    if (slot < 0 || slot >= num_slots) return;     // padding / out of range: no write
    const uint4* ks = key + i * row_chunks;
    const uint4* vs = value + i * row_chunks;
    uint4* kd = k_cache + slot * row_chunks;
    uint4* vd = v_cache + slot * row_chunks;
    for (int32_t ch = threadIdx.x; ch < row_chunks; ch += blockDim.x) {
        kd[ch] = ks[ch];
        vd[ch] = vs[ch];
    }
}

// The same write into an FP8 pool: each lane reads 8 values of the 16-bit row (16 bytes),
// widens them exactly to fp32 and writes their 8 E4M3 codes (8 bytes).
template <class S>
__device__ __forceinline__ uint2 to_fp8x8(uint4 x) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t b[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) b[e] = fp8x2_from(S::lo(w[e]), S::hi(w[e]));
    return make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
}

template <class S>
__global__ __launch_bounds__(256) void rc_quantize(const uint4* __restrict__ key,
                                                   const uint4* __restrict__ value,
                                                   const int64_t* __restrict__ slots,
                                                   uint2* __restrict__ k_cache,
                                                   uint2* __restrict__ v_cache, int64_t num_slots,
                                                   int32_t row_chunks) {
    const int64_t i = blockIdx.x;
    const int64_t slot = slots[i];
    if (slot < 0 || slot >= num_slots) return;
    const uint4* ks = key + i * row_chunks;
    const uint4* vs = value + i * row_chunks;
    uint2* kd = k_cache + slot * row_chunks;
    uint2* vd = v_cache + slot * row_chunks;
    for (int32_t ch = threadIdx.x; ch < row_chunks; ch += blockDim.x) {
        kd[ch] = to_fp8x8<S>(ks[ch]);
        vd[ch] = to_fp8x8<S>(vs[ch]);
    }
}

// The new token of sequence b (position L - 1) into the slot its table gives it, all KV
// heads: one work-group per sequence, lanes over the row's 32-bit words (two values).
// A sequence of length 0, or whose table entry names no block of the pool, writes
// nothing.  FP8 pools take the row rounded to E4M3 as in rc_quantize.
template <class S, bool KV8>
__global__ __launch_bounds__(256) void append_kv(DecodeArgs a) {
    const int b = blockIdx.x;
    const int L = clamped_length(a, b);
    if (L == 0) return;
    const int last = L - 1;
    const int blk = a.tables[static_cast<size_t>(b) * a.table_stride + last / a.block_size];
    if (static_cast<unsigned>(blk) >= static_cast<unsigned>(a.num_blocks)) return;
    const size_t slot = static_cast<size_t>(blk) * a.block_size + last % a.block_size;
    const int words = a.row_bytes / (KV8 ? 2 : 4);          // 32-bit words of the input row
    const uint32_t* ks = reinterpret_cast<const uint32_t*>(a.new_k) + static_cast<size_t>(b) * words;
    const uint32_t* vs = reinterpret_cast<const uint32_t*>(a.new_v) + static_cast<size_t>(b) * words;
    uint8_t* kd = const_cast<uint8_t*>(a.k) + slot * a.row_bytes;
    uint8_t* vd = const_cast<uint8_t*>(a.v) + slot * a.row_bytes;
    for (int w = threadIdx.x; w < words; w += blockDim.x) {
        if constexpr (KV8) {
            reinterpret_cast<uint16_t*>(kd)[w] = static_cast<uint16_t>(fp8x2_from(S::lo(ks[w]), S::hi(ks[w])));
            reinterpret_cast<uint16_t*>(vd)[w] = static_cast<uint16_t>(fp8x2_from(S::lo(vs[w]), S::hi(vs[w])));
        } else {
            reinterpret_cast<uint32_t*>(kd)[w] = ks[w];
            reinterpret_cast<uint32_t*>(vd)[w] = vs[w];
        }
    }
}

// One work-group per (table entry j, sequence b): the B rows of logical block j.
__global__ __launch_bounds__(256) void kv_gather(const uint4* __restrict__ k_cache,
                                                 const uint4* __restrict__ v_cache,
                                                 const int32_t* __restrict__ tables,
                                                 int32_t max_blocks,
                                                 const int32_t* __restrict__ lens,
                                                 int32_t num_blocks, int32_t block_size,
                                                 int32_t row_chunks, uint4* __restrict__ k_out,
                                                 uint4* __restrict__ v_out) {
    const int j = blockIdx.x;
    const int b = blockIdx.y;
    int L = lens[b];
    L = L < 0 ? 0 : (L > max_blocks * block_size ? max_blocks * block_size : L);
    const int valid = min(block_size, max(0, L - j * block_size));
    int blk = valid > 0 ? tables[static_cast<size_t>(b) * max_blocks + j] : -1;
    const bool ok = static_cast<unsigned>(blk) < static_cast<unsigned>(num_blocks);
    const size_t dst0 = (static_cast<size_t>(b) * max_blocks + j) * block_size * row_chunks;
    const size_t src0 = ok ? static_cast<size_t>(blk) * block_size * row_chunks : 0;
    const uint4 zero = make_uint4(0, 0, 0, 0);
    for (int idx = threadIdx.x; idx < block_size * row_chunks; idx += blockDim.x) {
        const int t = idx / row_chunks;
        const bool take = ok && t < valid;
        k_out[dst0 + idx] = take ? k_cache[src0 + idx] : zero;
        v_out[dst0 + idx] = take ? v_cache[src0 + idx] : zero;
    }
}

// Copy-on-write copies ("PagedAttention and Virtual Memory Management", section 5,
// case 2: the o token rows already in the shared block p go to the new block p_new).
// copies[i] = (src, dst, rows).  One work-group per (copy, layer, K or V): the first
// `rows` rows of a block are one contiguous stretch of rows * row_chunks 16-byte
// chunks, copied with coalesced dwordx4 accesses.  A triple with a block outside the
// pool, rows outside [0, block_size] or src == dst is skipped.
__global__ __launch_bounds__(256) void cow_copy(uint4* __restrict__ base,
                                                const int32_t* __restrict__ copies,
                                                int32_t num_blocks, int32_t block_size,
                                                int32_t row_chunks, size_t cache_chunks) {
    const int i = blockIdx.x;
    const int tensor = blockIdx.y;                   // 2 * layer + (0 for K, 1 for V)
    const int src = copies[3 * i + 0];
    const int dst = copies[3 * i + 1];
    const int rows = copies[3 * i + 2];
    if (static_cast<unsigned>(src) >= static_cast<unsigned>(num_blocks) ||
        static_cast<unsigned>(dst) >= static_cast<unsigned>(num_blocks) || src == dst ||
        rows <= 0 || rows > block_size)
        return;
    const size_t block_chunks = static_cast<size_t>(block_size) * row_chunks;
    const uint4* from = base + tensor * cache_chunks + static_cast<size_t>(src) * block_chunks;
    uint4* to = base + tensor * cache_chunks + static_cast<size_t>(dst) * block_chunks;
    const int n = rows * row_chunks;
    for (int ch = threadIdx.x; ch < n; ch += blockDim.x) to[ch] = from[ch];
}

// Swap copies between two pools of the same block shape, one or both in pinned host
// memory reached through its device mapping ("PagedAttention and Virtual Memory
// Management", section 6, swapping policy).  pairs[i] = (src block, dst block); every
// layer's K and V block is one contiguous stretch of block_chunks 16-byte chunks.
// Items are (tensor, pair) stretches, numbered pair-fastest so neighbouring items of one
// tensor follow the pair list (a run of consecutive blocks stays one run of addresses on
// the host link).  A fixed, small grid walks the items: the host link, not the CUs, is
// the limit, and the rest of the chip stays free for decode.  Each thread keeps kUnroll
// loads in flight before it stores, to cover the host link's latency.  A pair naming a
// block outside its pool is skipped.
constexpr int kSwapThreads = 256;
constexpr int kSwapUnroll = 4;

__global__ __launch_bounds__(kSwapThreads) void swap_copy(
    const uint4* __restrict__ src, uint4* __restrict__ dst, const int2* __restrict__ pairs,
    int32_t num_pairs, int64_t items, int32_t src_blocks, int32_t dst_blocks,
    int32_t block_chunks, size_t src_cache_chunks, size_t dst_cache_chunks) {
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int64_t tensor = it / num_pairs;
        const int2 pr = pairs[it - tensor * num_pairs];
        if (static_cast<unsigned>(pr.x) >= static_cast<unsigned>(src_blocks) ||
            static_cast<unsigned>(pr.y) >= static_cast<unsigned>(dst_blocks))
            continue;
        const uint4* from = src + tensor * src_cache_chunks + static_cast<size_t>(pr.x) * block_chunks;
        uint4* to = dst + tensor * dst_cache_chunks + static_cast<size_t>(pr.y) * block_chunks;
        for (int c0 = threadIdx.x; c0 < block_chunks; c0 += kSwapThreads * kSwapUnroll) {
            uint4 r[kSwapUnroll];
#pragma unroll
            for (int u = 0; u < kSwapUnroll; ++u) {
                const int c = c0 + u * kSwapThreads;
                if (c < block_chunks) r[u] = from[c];
            }
#pragma unroll
            for (int u = 0; u < kSwapUnroll; ++u) {
                const int c = c0 + u * kSwapThreads;
                if (c < block_chunks) to[c] = r[u];
            }
        }
    }
}

}  // namespace

hipError_t launch_append_kv(int kv_dtype, int io_dtype, const DecodeArgs& a, hipStream_t stream) {
    if (a.batch <= 0 || !a.new_k) return hipSuccess;
    const bool kv8 = kv_dtype == KV_DTYPE_FP8_E4M3;
    auto kernel = io_dtype == KV_DTYPE_F16 ? (kv8 ? append_kv<F16, true> : append_kv<F16, false>)
                                           : (kv8 ? append_kv<BF16, true> : append_kv<BF16, false>);
    hipLaunchKernelGGL(kernel, dim3(a.batch), dim3(256), 0, stream, a);
    return hipGetLastError();
}

int swap_groups() {
    static const int groups = [] {
        const char* e = getenv("PAGEDKV_SWAP_GROUPS");
        const int v = e ? atoi(e) : 0;
        return v > 0 && v <= 65535 ? v : kDefaultSwapGroups;
    }();
    return groups;
}

hipError_t launch_swap_blocks(const char* src, char* dst, const int32_t* pairs, int32_t num_pairs,
                              int32_t num_layers, int32_t src_blocks, int32_t dst_blocks,
                              size_t block_bytes, size_t src_cache_bytes, size_t dst_cache_bytes,
                              hipStream_t stream) {
    if (num_pairs <= 0) return hipSuccess;
    const int64_t items = static_cast<int64_t>(num_pairs) * 2 * num_layers;
    const int64_t groups = items < swap_groups() ? items : swap_groups();
    hipLaunchKernelGGL(swap_copy, dim3(static_cast<unsigned>(groups)), dim3(kSwapThreads), 0,
                       stream, reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst),
                       reinterpret_cast<const int2*>(pairs), num_pairs, items, src_blocks,
                       dst_blocks, static_cast<int32_t>(block_bytes / 16), src_cache_bytes / 16,
                       dst_cache_bytes / 16);
    return hipGetLastError();
}

hipError_t launch_copy_blocks(char* base, const int32_t* copies, int32_t num_copies,
                              int32_t num_layers, int32_t num_blocks, int32_t block_size,
                              int32_t row_bytes, size_t cache_bytes, hipStream_t stream) {
    if (num_copies <= 0) return hipSuccess;
    hipLaunchKernelGGL(cow_copy, dim3(num_copies, 2 * num_layers), dim3(256), 0, stream,
                       reinterpret_cast<uint4*>(base), copies, num_blocks, block_size,
                       row_bytes / 16, cache_bytes / 16);
    return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const void* key, const void* value, const int64_t* slots,
                                    int32_t num_tokens, void* k_cache, void* v_cache,
                                    int64_t num_slots, int32_t row_elems, int kv_dtype,
                                    int io_dtype, hipStream_t stream) {
    if (num_tokens <= 0) return hipSuccess;
    const int32_t chunks = row_elems / 8;          // 8 values: 16 input bytes
    const int threads = chunks >= 256 ? 256 : ((chunks + 63) / 64) * 64;
    const uint4* k = static_cast<const uint4*>(key);
    const uint4* v = static_cast<const uint4*>(value);
    if (kv_dtype == KV_DTYPE_FP8_E4M3) {
        auto kernel = io_dtype == KV_DTYPE_F16 ? rc_quantize<F16> : rc_quantize<BF16>;
        hipLaunchKernelGGL(kernel, dim3(num_tokens), dim3(threads), 0, stream, k, v, slots,
                           static_cast<uint2*>(k_cache), static_cast<uint2*>(v_cache), num_slots,
                           chunks);
    } else {
        hipLaunchKernelGGL(rc_scatter, dim3(num_tokens), dim3(threads), 0, stream, k, v, slots,
                           static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), num_slots,
                           chunks);
    }
    return hipGetLastError();
}

hipError_t launch_gather(const void* k_cache, const void* v_cache, const int32_t* tables,
                         int32_t max_blocks, const int32_t* lens, int32_t batch,
                         int32_t num_blocks, int32_t block_size, int32_t row_bytes,
                         void* k_out, void* v_out, hipStream_t stream) {
    if (batch <= 0 || max_blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(kv_gather, dim3(max_blocks, batch), dim3(256), 0, stream,
                       static_cast<const uint4*>(k_cache), static_cast<const uint4*>(v_cache),
                       tables, max_blocks, lens, num_blocks, block_size, row_bytes / 16,
                       static_cast<uint4*>(k_out), static_cast<uint4*>(v_out));
    return hipGetLastError();
}

}  // namespace pkv
