// Checked mode (PAGEDKV_CHECK=1): device pre-passes that validate the arguments the
// kernels only trust in the fast path, before anything is written.  Each sets bits of a
// device status word; the entry point then waits for the stream, reads the word, and
// returns KV_ERR_INVALID_ARG if any bit is set.  A debugging aid: it synchronises, so it
// is neither fast nor safe to capture in a graph.
//  * block tables: every entry a sequence uses (the first ceil(L / B)) names a block of
//    the pool, and every length is in [0, max_blocks * B] (the fast path clamps);
//  * slot mappings: every slot is below num_blocks * B (negative = no write, allowed) and
//    no slot appears twice (the fast path's result is then unspecified);
//  * query offsets (prefill): non-decreasing, chunk sizes within max_query_len;
//  * a shared prefix (decode over a forked prompt): every sequence's used entries among
//    the first prefix_blocks are row 0's, and a new token is never written into them.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "internal.h"

namespace pkv {
namespace {

constexpr uint32_t kBadBlock = 1u, kBadLength = 2u, kBadSlot = 4u, kDuplicateSlot = 8u,
                   kBadQueryStart = 16u, kBadPrefix = 32u;

__global__ __launch_bounds__(256) void check_shared_prefix(const int32_t* __restrict__ tables,
                                                           int32_t max_blocks,
                                                           const int32_t* __restrict__ lens,
                                                           int32_t batch, int32_t prefix_blocks,
                                                           int32_t block_size, int32_t appending,
                                                           uint32_t* status) {
    const int b = blockIdx.x;
    if (b >= batch) return;
    const int L = lens[b];
    uint32_t bad = 0;
    const int64_t prefix_len = static_cast<int64_t>(prefix_blocks) * block_size;
    if (appending && L > 0 && L <= prefix_len) bad |= kBadPrefix;
    const int used = L <= 0 ? 0 : min(prefix_blocks, (L + block_size - 1) / block_size);
    for (int j = threadIdx.x; j < used; j += blockDim.x)
        if (tables[static_cast<size_t>(b) * max_blocks + j] != tables[j]) bad |= kBadPrefix;
    if (bad) atomicOr(status, bad);
}

__global__ __launch_bounds__(256) void check_tables(const int32_t* __restrict__ tables, int32_t max_blocks,
                                                    const int32_t* __restrict__ lens, int32_t batch,
                                                    int32_t num_blocks, int32_t block_size,
                                                    uint32_t* status) {
    const int b = blockIdx.x;
    if (b >= batch) return;
    const int L = lens[b];
    uint32_t bad = 0;
    if (L < 0 || static_cast<int64_t>(L) > static_cast<int64_t>(max_blocks) * block_size) bad |= kBadLength;
    const int used = L <= 0 ? 0 : min(max_blocks, (L + block_size - 1) / block_size);
    for (int j = threadIdx.x; j < used; j += blockDim.x) {
        const int t = tables[static_cast<size_t>(b) * max_blocks + j];
        if (static_cast<unsigned>(t) >= static_cast<unsigned>(num_blocks)) bad |= kBadBlock;
    }
    if (bad) atomicOr(status, bad);
}

__global__ __launch_bounds__(256) void clear_words(uint32_t* w, int64_t n) {
    for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        w[i] = 0u;
}

// one bit per slot of the layer: a slot seen twice finds its bit already set
__global__ __launch_bounds__(256) void check_slots(const int64_t* __restrict__ slots, int32_t n,
                                                   int64_t num_slots, uint32_t* seen, uint32_t* status) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int64_t s = slots[i];
    if (s < 0) return;
    if (s >= num_slots) {
        atomicOr(status, kBadSlot);
        return;
    }
    const uint32_t bit = 1u << (s & 31);
    if (atomicOr(seen + (s >> 5), bit) & bit) atomicOr(status, kDuplicateSlot);
}

// the decode-with-append slots: position L - 1 of each sequence, through its table; two
// sequences whose new tokens land in one slot find its bit already set (lengths and
// block ids are check_tables' part)
__global__ __launch_bounds__(256) void check_append_slots(const int32_t* __restrict__ tables,
                                                          int32_t max_blocks,
                                                          const int32_t* __restrict__ lens,
                                                          int32_t batch, int32_t num_blocks,
                                                          int32_t block_size, uint32_t* seen,
                                                          uint32_t* status) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= batch) return;
    const int L = lens[b];
    if (L <= 0 || static_cast<int64_t>(L) > static_cast<int64_t>(max_blocks) * block_size) return;
    const int blk = tables[static_cast<size_t>(b) * max_blocks + (L - 1) / block_size];
    if (static_cast<unsigned>(blk) >= static_cast<unsigned>(num_blocks)) return;
    const int64_t s = static_cast<int64_t>(blk) * block_size + (L - 1) % block_size;
    const uint32_t bit = 1u << (s & 31);
    if (atomicOr(seen + (s >> 5), bit) & bit) atomicOr(status, kDuplicateSlot);
}

__global__ __launch_bounds__(256) void check_query_start(const int32_t* __restrict__ qs, int32_t batch,
                                                         int32_t max_query_len, uint32_t* status) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= batch) return;
    const int n = qs[b + 1] - qs[b];
    if (qs[b] < 0 || n < 0 || n > max_query_len) atomicOr(status, kBadQueryStart);
}

}  // namespace

hipError_t launch_check_tables(const int32_t* tables, int32_t max_blocks, const int32_t* lens,
                               int32_t batch, int32_t num_blocks, int32_t block_size,
                               uint32_t* status, hipStream_t stream) {
    if (batch <= 0) return hipSuccess;
    hipLaunchKernelGGL(check_tables, dim3(batch), dim3(256), 0, stream, tables, max_blocks, lens,
                       batch, num_blocks, block_size, status);
    return hipGetLastError();
}

hipError_t launch_check_slots(const int64_t* slots, int32_t n, int64_t num_slots, uint32_t* seen,
                              uint32_t* status, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t words = (num_slots + 31) / 32;
    hipLaunchKernelGGL(clear_words, dim3(static_cast<unsigned>(std::min<int64_t>((words + 255) / 256, 4096))),
                       dim3(256), 0, stream, seen, words);
    hipLaunchKernelGGL(check_slots, dim3((n + 255) / 256), dim3(256), 0, stream, slots, n, num_slots,
                       seen, status);
    return hipGetLastError();
}

hipError_t launch_check_shared_prefix(const int32_t* tables, int32_t max_blocks, const int32_t* lens,
                                      int32_t batch, int32_t prefix_blocks, int32_t block_size,
                                      int32_t appending, uint32_t* status, hipStream_t stream) {
    if (batch <= 0) return hipSuccess;
    hipLaunchKernelGGL(check_shared_prefix, dim3(batch), dim3(256), 0, stream, tables, max_blocks,
                       lens, batch, prefix_blocks, block_size, appending, status);
    return hipGetLastError();
}

hipError_t launch_check_append_slots(const int32_t* tables, int32_t max_blocks, const int32_t* lens,
                                     int32_t batch, int32_t num_blocks, int32_t block_size,
                                     uint32_t* seen, uint32_t* status, hipStream_t stream) {
    if (batch <= 0) return hipSuccess;
    const int64_t words = (static_cast<int64_t>(num_blocks) * block_size + 31) / 32;
    hipLaunchKernelGGL(clear_words, dim3(static_cast<unsigned>(std::min<int64_t>((words + 255) / 256, 4096))),
                       dim3(256), 0, stream, seen, words);
    hipLaunchKernelGGL(check_append_slots, dim3((batch + 255) / 256), dim3(256), 0, stream, tables,
                       max_blocks, lens, batch, num_blocks, block_size, seen, status);
    return hipGetLastError();
}

hipError_t launch_check_query_start(const int32_t* qs, int32_t batch, int32_t max_query_len,
                                    uint32_t* status, hipStream_t stream) {
    if (batch <= 0) return hipSuccess;
    hipLaunchKernelGGL(check_query_start, dim3((batch + 255) / 256), dim3(256), 0, stream, qs, batch,
                       max_query_len, status);
    return hipGetLastError();
}

hipError_t launch_clear_word(uint32_t* w, hipStream_t stream) {
    hipLaunchKernelGGL(clear_words, dim3(1), dim3(64), 0, stream, w, int64_t(1));
    return hipGetLastError();
}

}  // namespace pkv
