// Host block manager: the free list, reference counts and per-request block tables that
// decide where each new token's key and value go, plus the copy-on-write copies a
// decode step needs.  The device side of a step is then kv_copy_blocks (the copies),
// reshape_and_cache (the slots) and paged_attention_decode (the exported tables).
//
// Behaviour follows "Why AI servers waste memory, and how paging fixes it" ("The idea:
// a block table", "A hand-worked example", "The real implementation", "Sharing a prefix
// with copy-on-write") and section 5 of "PagedAttention and Virtual Memory Management"
// (reference counts; a write into a shared block allocates a new block, copies the o
// rows already written, drops the old block's count and repoints the table):
//  * new blocks come from the front of the free list, freed blocks join its back;
//  * a request that stores a token at a block boundary takes a new block; one whose
//    last block is shared with another request and still has room takes a new block
//    and reports the copy (src, dst, rows = length mod B);
//  * fork copies the parent's table and adds one reference to each block it names;
//  * free drops one reference per block, front to back, and returns a block to the
//    free list when no table names it any more;
//  * every call checks everything it needs before it changes anything, so a call that
//    fails (no free block, unknown request) leaves the manager as it was.
//
// Data layout: the free list is a ring buffer over all block ids (O(1) take and give
// back), reference counts a dense array, and tables vectors in a hash map keyed by the
// caller's 64-bit request id.  Not thread-safe: one caller at a time.

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

struct kv_block_manager {
    int32_t num_blocks;
    int32_t block_size;
    std::vector<int32_t> ring;     // free block ids, ring[(head + i) % num_blocks], i < num_free
    int32_t head;
    int32_t num_free;
    std::vector<int32_t> refs;
    struct Request {
        std::vector<int32_t> table;
        int32_t length;
    };
    std::unordered_map<int64_t, Request> requests;

    int32_t take() {
        const int32_t b = ring[head];
        head = head + 1 == num_blocks ? 0 : head + 1;
        --num_free;
        refs[b] = 1;
        return b;
    }
    void give_back(int32_t b) {
        int64_t tail = static_cast<int64_t>(head) + num_free;
        if (tail >= num_blocks) tail -= num_blocks;
        ring[tail] = b;
        ++num_free;
    }
};

namespace {

// Blocks a batch of appends takes, simulated without changing anything; -1 if a request
// id is unknown or a count is negative.  Shared blocks can become private during the
// batch (a copy drops the old block's count), so counts are tracked as deltas.
int64_t blocks_needed(const kv_block_manager& m, const int64_t* rids, const int32_t* counts,
                      int32_t n) {
    std::unordered_map<int64_t, std::pair<int32_t, int32_t>> local;   // rid -> (length, last)
    std::unordered_map<int32_t, int32_t> delta;                      // block -> ref change
    int64_t need = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t c = counts ? counts[i] : 1;
        auto it = m.requests.find(rids[i]);
        if (c < 0 || it == m.requests.end()) return -1;
        auto lt = local.find(rids[i]);
        int32_t len = lt != local.end() ? lt->second.first : it->second.length;
        int32_t last = lt != local.end() ? lt->second.second
                                         : (it->second.table.empty() ? -1 : it->second.table.back());
        for (int32_t t = 0; t < c; ++t) {
            const int32_t offset = len % m.block_size;
            if (offset == 0) {
                ++need;
                last = -1;                     // a fresh block: owned alone
            } else if (last >= 0) {
                auto d = delta.find(last);
                const int32_t r = m.refs[last] + (d != delta.end() ? d->second : 0);
                if (r > 1) {
                    ++need;
                    delta[last] -= 1;
                    last = -1;
                }
            }
            ++len;
        }
        local[rids[i]] = {len, last};
    }
    return need;
}

}  // namespace

extern "C" {

kv_status_t kv_bm_create(int32_t num_blocks, int32_t block_size, kv_block_manager_t** out) {
    if (num_blocks < 1 || block_size < 1 || !out) return KV_ERR_INVALID_ARG;
    kv_block_manager* m = new (std::nothrow) kv_block_manager();
    if (!m) return KV_ERR_OUT_OF_MEMORY;
    try {
        m->ring.resize(num_blocks);
        m->refs.assign(num_blocks, 0);
    } catch (...) {
        delete m;
        return KV_ERR_OUT_OF_MEMORY;
    }
    m->num_blocks = num_blocks;
    m->block_size = block_size;
    for (int32_t b = 0; b < num_blocks; ++b) m->ring[b] = b;
    m->head = 0;
    m->num_free = num_blocks;
    *out = m;
    return KV_OK;
}

kv_status_t kv_bm_destroy(kv_block_manager_t* m) {
    delete m;
    return KV_OK;
}

kv_status_t kv_bm_add_request(kv_block_manager_t* m, int64_t rid) {
    if (!m || m->requests.count(rid)) return KV_ERR_INVALID_ARG;
    try {
        m->requests.emplace(rid, kv_block_manager::Request{{}, 0});
    } catch (...) {
        return KV_ERR_OUT_OF_MEMORY;
    }
    return KV_OK;
}

kv_status_t kv_bm_fork(kv_block_manager_t* m, int64_t parent, int64_t child) {
    if (!m || m->requests.count(child)) return KV_ERR_INVALID_ARG;
    auto it = m->requests.find(parent);
    if (it == m->requests.end()) return KV_ERR_INVALID_ARG;
    try {
        kv_block_manager::Request copy = it->second;
        m->requests.emplace(child, std::move(copy));
    } catch (...) {
        return KV_ERR_OUT_OF_MEMORY;
    }
    for (int32_t b : m->requests[child].table) ++m->refs[b];
    return KV_OK;
}

kv_status_t kv_bm_free_request(kv_block_manager_t* m, int64_t rid) {
    if (!m) return KV_ERR_INVALID_ARG;
    auto it = m->requests.find(rid);
    if (it == m->requests.end()) return KV_ERR_INVALID_ARG;
    for (int32_t b : it->second.table)
        if (--m->refs[b] == 0) m->give_back(b);
    m->requests.erase(it);
    return KV_OK;
}

kv_status_t kv_bm_append(kv_block_manager_t* m, const int64_t* rids, const int32_t* counts,
                         int32_t n, int64_t* slots, int64_t slots_cap, int32_t* copies,
                         int32_t copies_cap, int32_t* num_copies) {
    if (!m || n < 0 || (n > 0 && !rids) || !num_copies) return KV_ERR_INVALID_ARG;
    int64_t total = 0;
    for (int32_t i = 0; i < n; ++i) total += counts ? counts[i] : 1;
    if (total > 0 && (!slots || slots_cap < total)) return KV_ERR_INVALID_ARG;
    const int64_t need = blocks_needed(*m, rids, counts, n);
    if (need < 0) return KV_ERR_INVALID_ARG;
    if (need > m->num_free) return KV_ERR_OUT_OF_BLOCKS;
    // copies: at most one per request occurrence (only a request's first token of the
    // batch can find its last block shared)
    int32_t ncopy_max = 0;
    for (int32_t i = 0; i < n; ++i) ncopy_max += (counts ? counts[i] : 1) > 0 ? 1 : 0;
    if (ncopy_max > 0 && (!copies || copies_cap < ncopy_max)) return KV_ERR_INVALID_ARG;
    // make room in the tables first, so that nothing below can fail half-way
    try {
        for (int32_t i = 0; i < n; ++i) {
            auto& r = m->requests[rids[i]];
            const int64_t c = counts ? counts[i] : 1;
            r.table.reserve(r.table.size() + static_cast<size_t>(c / m->block_size + 1));
        }
    } catch (...) {
        return KV_ERR_OUT_OF_MEMORY;
    }
    int64_t s = 0;
    int32_t nc = 0;
    for (int32_t i = 0; i < n; ++i) {
        auto& r = m->requests[rids[i]];
        const int32_t c = counts ? counts[i] : 1;
        for (int32_t t = 0; t < c; ++t) {
            const int32_t offset = r.length % m->block_size;
            if (offset == 0) {
                r.table.push_back(m->take());
            } else if (m->refs[r.table.back()] > 1) {
                const int32_t old = r.table.back();
                const int32_t fresh = m->take();
                --m->refs[old];
                r.table.back() = fresh;
                copies[3 * nc + 0] = old;
                copies[3 * nc + 1] = fresh;
                copies[3 * nc + 2] = offset;
                ++nc;
            }
            slots[s++] = static_cast<int64_t>(r.table.back()) * m->block_size + offset;
            ++r.length;
        }
    }
    *num_copies = nc;
    return KV_OK;
}

kv_status_t kv_bm_get_length(const kv_block_manager_t* m, int64_t rid, int32_t* length) {
    if (!m || !length) return KV_ERR_INVALID_ARG;
    auto it = m->requests.find(rid);
    if (it == m->requests.end()) return KV_ERR_INVALID_ARG;
    *length = it->second.length;
    return KV_OK;
}

kv_status_t kv_bm_get_table(const kv_block_manager_t* m, int64_t rid, int32_t* table,
                            int32_t cap, int32_t* num) {
    if (!m || !num) return KV_ERR_INVALID_ARG;
    auto it = m->requests.find(rid);
    if (it == m->requests.end()) return KV_ERR_INVALID_ARG;
    const auto& t = it->second.table;
    const int32_t size = static_cast<int32_t>(t.size());
    if (size > 0 && (!table || cap < size)) return KV_ERR_INVALID_ARG;
    if (size > 0) memcpy(table, t.data(), sizeof(int32_t) * size);
    *num = size;
    return KV_OK;
}

kv_status_t kv_bm_export(const kv_block_manager_t* m, const int64_t* rids, int32_t n,
                         int32_t max_blocks, int32_t* tables, int32_t* lengths) {
    if (!m || n < 0 || max_blocks < 1) return KV_ERR_INVALID_ARG;
    if (n == 0) return KV_OK;
    if (!rids || !tables || !lengths) return KV_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n; ++i) {            // check everything before writing
        auto it = m->requests.find(rids[i]);
        if (it == m->requests.end() || static_cast<int64_t>(it->second.table.size()) > max_blocks)
            return KV_ERR_INVALID_ARG;
    }
    for (int32_t i = 0; i < n; ++i) {
        const auto& r = m->requests.find(rids[i])->second;
        int32_t* row = tables + static_cast<size_t>(i) * max_blocks;
        const int32_t size = static_cast<int32_t>(r.table.size());
        if (size > 0) memcpy(row, r.table.data(), sizeof(int32_t) * size);
        for (int32_t j = size; j < max_blocks; ++j) row[j] = -1;
        lengths[i] = r.length;
    }
    return KV_OK;
}

kv_status_t kv_bm_move(kv_block_manager_t* src, kv_block_manager_t* dst, const int64_t* rids,
                       int32_t n, int32_t* pairs, int32_t pairs_cap, int32_t* num_pairs) {
    if (!src || !dst || src == dst || n < 0 || (n > 0 && !rids) || !num_pairs ||
        src->block_size != dst->block_size)
        return KV_ERR_INVALID_ARG;
    // check everything first: ids known here, new there, not repeated; room for the pairs
    std::unordered_map<int32_t, int32_t> fresh;          // source block -> destination block
    std::vector<int32_t> order;                          // distinct source blocks, first seen
    try {
        std::unordered_map<int64_t, int> seen;
        for (int32_t i = 0; i < n; ++i) {
            auto it = src->requests.find(rids[i]);
            if (it == src->requests.end() || dst->requests.count(rids[i]) || seen[rids[i]]++)
                return KV_ERR_INVALID_ARG;
            for (int32_t b : it->second.table)
                if (fresh.emplace(b, -1).second) order.push_back(b);
        }
        dst->requests.reserve(dst->requests.size() + n);
    } catch (...) {
        return KV_ERR_OUT_OF_MEMORY;
    }
    const int32_t need = static_cast<int32_t>(order.size());
    if (need > 0 && (!pairs || pairs_cap < need)) return KV_ERR_INVALID_ARG;
    if (need > dst->num_free) return KV_ERR_OUT_OF_BLOCKS;
    // the destination's requests first (copies of the tables, so nothing below can fail)
    std::vector<kv_block_manager::Request> moved;
    try {
        moved.reserve(n);
        for (int32_t i = 0; i < n; ++i) moved.push_back(src->requests.find(rids[i])->second);
    } catch (...) {
        return KV_ERR_OUT_OF_MEMORY;
    }
    for (int32_t k = 0; k < need; ++k) {
        const int32_t b = dst->take();
        dst->refs[b] = 0;                               // counted from the tables below
        fresh[order[k]] = b;
        pairs[2 * k + 0] = order[k];
        pairs[2 * k + 1] = b;
    }
    for (int32_t i = 0; i < n; ++i) {
        for (int32_t& b : moved[i].table) {
            b = fresh[b];
            ++dst->refs[b];
        }
        dst->requests.emplace(rids[i], std::move(moved[i]));
    }
    for (int32_t i = 0; i < n; ++i) kv_bm_free_request(src, rids[i]);
    *num_pairs = need;
    return KV_OK;
}

int32_t kv_bm_num_free(const kv_block_manager_t* m) { return m ? m->num_free : -1; }

kv_status_t kv_bm_ref_count(const kv_block_manager_t* m, int32_t block, int32_t* count) {
    if (!m || !count || block < 0 || block >= m->num_blocks) return KV_ERR_INVALID_ARG;
    *count = m->refs[block];
    return KV_OK;
}

kv_status_t kv_bm_free_list(const kv_block_manager_t* m, int32_t* blocks, int32_t cap,
                            int32_t* num) {
    if (!m || !num) return KV_ERR_INVALID_ARG;
    if (m->num_free > 0 && (!blocks || cap < m->num_free)) return KV_ERR_INVALID_ARG;
    for (int32_t i = 0; i < m->num_free; ++i) {
        int64_t k = static_cast<int64_t>(m->head) + i;
        if (k >= m->num_blocks) k -= m->num_blocks;
        blocks[i] = m->ring[k];
    }
    *num = m->num_free;
    return KV_OK;
}

// The largest prefix the shared-prefix decode accepts for these host tables (see
// include/pagedkv.h): row 0's leading blocks, cut at the first entry a sequence uses
// that differs from row 0's, and with new tokens before each sequence's last position.
int32_t kv_shared_prefix_blocks(const int32_t* tables, const int32_t* lengths, int32_t batch,
                                int32_t max_blocks, int32_t block_size, int32_t appending) {
    if (!tables || !lengths || batch < 1 || max_blocks < 1 ||
        (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64))
        return -1;
    auto used = [&](int32_t b) -> int32_t {      // entries sequence b's length reaches
        const int64_t L = std::min<int64_t>(std::max<int32_t>(lengths[b], 0),
                                            static_cast<int64_t>(max_blocks) * block_size);
        return static_cast<int32_t>((L + block_size - 1) / block_size);
    };
    int32_t p = 0;                               // row 0's leading blocks
    while (p < max_blocks && tables[p] >= 0) ++p;
    for (int32_t b = 1; b < batch && p > 0; ++b) {
        const int32_t* row = tables + static_cast<size_t>(b) * max_blocks;
        const int32_t n = std::min(p, used(b));
        int32_t j = 0;
        while (j < n && row[j] == tables[j]) ++j;
        if (j < n) p = j;                        // a used entry differs from row 0's
    }
    if (appending) {
        for (int32_t b = 0; b < batch && p > 0; ++b) {
            const int32_t L = std::min<int64_t>(lengths[b], static_cast<int64_t>(max_blocks) * block_size);
            if (L > 0) p = std::min(p, (L - 1) / block_size);
        }
    }
    return p;
}

// A batch order for a decode step: the sequences by length, longest first, ties in batch
// order (see include/pagedkv.h).
int32_t kv_decode_order(const int32_t* lengths, int32_t batch, int32_t* order) {
    if (!lengths || !order || batch < 0) return -1;
    for (int32_t i = 0; i < batch; ++i) order[i] = i;
    std::stable_sort(order, order + batch, [&](int32_t x, int32_t y) { return lengths[x] > lengths[y]; });
    return 0;
}

}  // extern "C"
