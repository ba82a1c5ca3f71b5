// Host-side automatic prefix caching on a paged block pool: which physical blocks a new
// request can reuse because an earlier request already computed the same prefix.
//
// Behaviour ("PagedAttention: Treating KV Memory Like Virtual Memory", "A separate
// mechanism: automatic prefix caching"; "2.1 PagedAttention", section 9):
//  * a block is hashed when it fills up, from the previous block's hash, its token ids
//    and, for a request's first block, the request's salt: the hashes form a chain, so a
//    hit means agreement from the first token, and a match ends on a block boundary;
//  * a new request finds the leading full blocks of its prompt in the hash table; a hit
//    copies nothing and raises the block's count (a free cached block leaves the free
//    queue);
//  * finishing lowers the counts of the request's blocks, last block first; blocks that
//    reach zero return to the free queue with their hash intact, hash-less ones at the
//    head (reused first) and cached ones at the tail (evicted last, oldest first);
//  * taking a cached free block for new data evicts its hash; a call that cannot get
//    enough blocks fails before it changes anything.
// The hash is 64-bit FNV-1a over the little-endian bytes of (previous hash, token ids,
// salt on the first block).
//
// Data layout: the free queue is a doubly linked list threaded through two int32 arrays
// (O(1) take at the head, insert at either end, removal from the middle on a hit); the
// hash table maps 64-bit hashes to blocks; each request keeps its table, its length, the
// token ids of its unfilled last block and the hash of its last full block.  Not
// thread-safe: one caller at a time.

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pagedkv.h"

namespace {

constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

uint64_t fnv_bytes(uint64_t h, const void* data, size_t n) {
    const unsigned char* p = static_cast<const unsigned char*>(data);
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= kFnvPrime;
    }
    return h;
}

// hash of one full block; host byte order is little-endian on every supported machine
uint64_t chain_hash(uint64_t prev, const int32_t* tokens, int32_t n, bool first, uint64_t salt) {
    uint64_t h = fnv_bytes(kFnvOffset, &prev, sizeof(prev));
    h = fnv_bytes(h, tokens, sizeof(int32_t) * static_cast<size_t>(n));
    if (first) h = fnv_bytes(h, &salt, sizeof(salt));
    return h;
}

}  // namespace

struct kv_prefix_cache {
    int32_t num_blocks;
    int32_t block_size;
    std::vector<int32_t> ref;
    std::vector<uint64_t> hash;
    std::vector<uint8_t> hashed;
    std::vector<int32_t> prev, next;     // free queue links (-1 = none)
    std::vector<uint8_t> in_free;
    int32_t head = -1, tail = -1, num_free = 0;
    std::unordered_map<uint64_t, int32_t> cached;
    struct Request {
        std::vector<int32_t> table;
        int32_t length = 0;
        std::vector<int32_t> partial;    // token ids of the unfilled last block
        uint64_t salt = 0;
        uint64_t last_hash = 0;          // hash of the last full block (0 before the first)
    };
    std::unordered_map<int64_t, Request> requests;

    void unlink(int32_t b) {
        const int32_t p = prev[b], n = next[b];
        if (p >= 0) next[p] = n; else head = n;
        if (n >= 0) prev[n] = p; else tail = p;
        prev[b] = next[b] = -1;
        in_free[b] = 0;
        --num_free;
    }
    void push_back(int32_t b) {
        prev[b] = tail;
        next[b] = -1;
        if (tail >= 0) next[tail] = b; else head = b;
        tail = b;
        in_free[b] = 1;
        ++num_free;
    }
    // insert b before `before` (-1: at the tail)
    void insert_before(int32_t b, int32_t before) {
        if (before < 0) {
            push_back(b);
            return;
        }
        const int32_t p = prev[before];
        prev[b] = p;
        next[b] = before;
        prev[before] = b;
        if (p >= 0) next[p] = b; else head = b;
        in_free[b] = 1;
        ++num_free;
    }
    int32_t take() {
        const int32_t b = head;
        unlink(b);
        if (hashed[b]) {                 // a cached free block: its hash is evicted
            cached.erase(hash[b]);
            hashed[b] = 0;
        }
        ref[b] = 1;
        return b;
    }
    // the request's next token: its slot; a block that fills up is hashed and cached (if
    // the hash is new; a failed insertion only leaves the block uncached).  The caller
    // has checked that a free block is there if one is needed and reserved the vectors.
    int64_t append_one(Request& r, int32_t token) {
        const int32_t B = block_size;
        const int32_t off = r.length % B;
        if (off == 0) r.table.push_back(take());
        const int32_t blk = r.table.back();
        r.partial.push_back(token);
        ++r.length;
        if (off + 1 == B) {
            const bool first = r.length == B;
            const uint64_t h = chain_hash(r.last_hash, r.partial.data(), B, first, r.salt);
            r.last_hash = h;
            r.partial.clear();
            if (!hashed[blk] && cached.find(h) == cached.end()) {
                try {
                    cached.emplace(h, blk);
                    hash[blk] = h;
                    hashed[blk] = 1;
                } catch (...) {
                }
            }
        }
        return static_cast<int64_t>(blk) * B + off;
    }
};

// room for `size` entries, growing the capacity geometrically (appends one block at a
// time stay amortised O(1)); may throw before anything else changes
void grow(std::vector<int32_t>& v, size_t size) {
    if (size > v.capacity()) v.reserve(std::max(size, 2 * v.capacity()));
}

extern "C" {

kv_status_t kv_pc_create(int32_t num_blocks, int32_t block_size, kv_prefix_cache_t** out) {
    if (num_blocks < 1 || block_size < 1 || !out) return KV_ERR_INVALID_ARG;
    kv_prefix_cache* pc = new (std::nothrow) kv_prefix_cache();
    if (!pc) return KV_ERR_OUT_OF_MEMORY;
    try {
        pc->ref.assign(num_blocks, 0);
        pc->hash.assign(num_blocks, 0);
        pc->hashed.assign(num_blocks, 0);
        pc->prev.assign(num_blocks, -1);
        pc->next.assign(num_blocks, -1);
        pc->in_free.assign(num_blocks, 0);
    } catch (...) {
        delete pc;
        return KV_ERR_OUT_OF_MEMORY;
    }
    pc->num_blocks = num_blocks;
    pc->block_size = block_size;
    for (int32_t b = 0; b < num_blocks; ++b) pc->push_back(b);
    *out = pc;
    return KV_OK;
}

kv_status_t kv_pc_destroy(kv_prefix_cache_t* pc) {
    delete pc;
    return KV_OK;
}

kv_status_t kv_pc_add_request(kv_prefix_cache_t* pc, int64_t rid, const int32_t* prompt,
                              int32_t n, uint64_t salt, int32_t* found_tokens) {
    if (!pc || n < 0 || (n > 0 && !prompt) || !found_tokens || pc->requests.count(rid))
        return KV_ERR_INVALID_ARG;
    const int32_t B = pc->block_size;
    std::vector<int32_t> matched;
    uint64_t h = 0;
    try {
        for (int32_t j = 0; j < n / B; ++j) {
            const uint64_t hj = chain_hash(h, prompt + static_cast<size_t>(j) * B, B, j == 0, salt);
            auto it = pc->cached.find(hj);
            if (it == pc->cached.end()) break;
            matched.push_back(it->second);
            h = hj;
        }
        kv_prefix_cache::Request r;
        r.table = matched;
        r.length = static_cast<int32_t>(matched.size()) * B;
        r.salt = salt;
        r.last_hash = h;
        r.table.reserve(matched.size() + 1);
        pc->requests.emplace(rid, std::move(r));
    } catch (...) {
        return KV_ERR_OUT_OF_MEMORY;
    }
    for (int32_t b : matched) {          // touch: hits leave the free queue
        if (pc->ref[b] == 0) pc->unlink(b);
        ++pc->ref[b];
    }
    *found_tokens = static_cast<int32_t>(matched.size()) * B;
    return KV_OK;
}

kv_status_t kv_pc_append(kv_prefix_cache_t* pc, int64_t rid, const int32_t* tokens, int32_t n,
                         int64_t* slots, int64_t slots_cap) {
    if (!pc || n < 0) return KV_ERR_INVALID_ARG;
    auto it = pc->requests.find(rid);
    if (it == pc->requests.end()) return KV_ERR_INVALID_ARG;
    if (n == 0) return KV_OK;
    if (!tokens || !slots || slots_cap < n) return KV_ERR_INVALID_ARG;
    auto& r = it->second;
    const int32_t B = pc->block_size;
    const int64_t have = (static_cast<int64_t>(r.length) + B - 1) / B;
    const int64_t want = (static_cast<int64_t>(r.length) + n + B - 1) / B;
    if (want - have > pc->num_free) return KV_ERR_OUT_OF_BLOCKS;
    try {
        grow(r.table, static_cast<size_t>(want));
        r.partial.reserve(static_cast<size_t>(B));
    } catch (...) {
        return KV_ERR_OUT_OF_MEMORY;
    }
    for (int32_t i = 0; i < n; ++i) slots[i] = pc->append_one(r, tokens[i]);
    return KV_OK;
}

kv_status_t kv_pc_append_step(kv_prefix_cache_t* pc, const int64_t* rids, const int32_t* tokens,
                              int32_t n, int64_t* slots) {
    if (!pc || n < 0) return KV_ERR_INVALID_ARG;
    if (n == 0) return KV_OK;
    if (!rids || !tokens || !slots) return KV_ERR_INVALID_ARG;
    const int32_t B = pc->block_size;
    std::vector<kv_prefix_cache::Request*> rs;
    int64_t need = 0;
    try {
        rs.reserve(static_cast<size_t>(n));
        std::unordered_set<int64_t> seen;
        seen.reserve(static_cast<size_t>(n));
        for (int32_t i = 0; i < n; ++i) {
            auto it = pc->requests.find(rids[i]);
            if (it == pc->requests.end() || !seen.insert(rids[i]).second) return KV_ERR_INVALID_ARG;
            auto& r = it->second;
            if (r.length % B == 0) {
                ++need;
                grow(r.table, r.table.size() + 1);
            }
            r.partial.reserve(static_cast<size_t>(B));
            rs.push_back(&r);
        }
    } catch (...) {
        return KV_ERR_OUT_OF_MEMORY;
    }
    if (need > pc->num_free) return KV_ERR_OUT_OF_BLOCKS;
    for (int32_t i = 0; i < n; ++i) slots[i] = pc->append_one(*rs[i], tokens[i]);
    return KV_OK;
}

kv_status_t kv_pc_free_request(kv_prefix_cache_t* pc, int64_t rid) {
    if (!pc) return KV_ERR_INVALID_ARG;
    auto it = pc->requests.find(rid);
    if (it == pc->requests.end()) return KV_ERR_INVALID_ARG;
    const std::vector<int32_t>& t = it->second.table;
    // last block first; of the blocks that reach zero, hash-less ones go to the head as a
    // group (in this order) and cached ones to the tail
    std::vector<int32_t> no_hash, has_hash;
    try {
        no_hash.reserve(t.size());
        has_hash.reserve(t.size());
    } catch (...) {
        return KV_ERR_OUT_OF_MEMORY;
    }
    for (size_t k = t.size(); k-- > 0;) {
        const int32_t b = t[k];
        if (--pc->ref[b] != 0) continue;
        (pc->hashed[b] ? has_hash : no_hash).push_back(b);
    }
    const int32_t old_head = pc->head;
    for (int32_t b : no_hash) pc->insert_before(b, old_head);
    for (int32_t b : has_hash) pc->push_back(b);
    pc->requests.erase(it);
    return KV_OK;
}

kv_status_t kv_pc_get_length(const kv_prefix_cache_t* pc, int64_t rid, int32_t* length) {
    if (!pc || !length) return KV_ERR_INVALID_ARG;
    auto it = pc->requests.find(rid);
    if (it == pc->requests.end()) return KV_ERR_INVALID_ARG;
    *length = it->second.length;
    return KV_OK;
}

kv_status_t kv_pc_get_table(const kv_prefix_cache_t* pc, int64_t rid, int32_t* table, int32_t cap,
                            int32_t* num) {
    if (!pc || !num) return KV_ERR_INVALID_ARG;
    auto it = pc->requests.find(rid);
    if (it == pc->requests.end()) return KV_ERR_INVALID_ARG;
    const auto& t = it->second.table;
    const int32_t size = static_cast<int32_t>(t.size());
    if (size > 0 && (!table || cap < size)) return KV_ERR_INVALID_ARG;
    if (size > 0) memcpy(table, t.data(), sizeof(int32_t) * size);
    *num = size;
    return KV_OK;
}

kv_status_t kv_pc_export(const kv_prefix_cache_t* pc, const int64_t* rids, int32_t n,
                         int32_t max_blocks, int32_t* tables, int32_t* lengths) {
    if (!pc || n < 0 || max_blocks < 1) return KV_ERR_INVALID_ARG;
    if (n == 0) return KV_OK;
    if (!rids || !tables || !lengths) return KV_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n; ++i) {
        auto it = pc->requests.find(rids[i]);
        if (it == pc->requests.end() || static_cast<int64_t>(it->second.table.size()) > max_blocks)
            return KV_ERR_INVALID_ARG;
    }
    for (int32_t i = 0; i < n; ++i) {
        const auto& r = pc->requests.find(rids[i])->second;
        int32_t* row = tables + static_cast<size_t>(i) * max_blocks;
        const int32_t size = static_cast<int32_t>(r.table.size());
        if (size > 0) memcpy(row, r.table.data(), sizeof(int32_t) * size);
        for (int32_t j = size; j < max_blocks; ++j) row[j] = -1;
        lengths[i] = r.length;
    }
    return KV_OK;
}

int32_t kv_pc_num_free(const kv_prefix_cache_t* pc) { return pc ? pc->num_free : -1; }

int32_t kv_pc_num_cached(const kv_prefix_cache_t* pc) {
    return pc ? static_cast<int32_t>(pc->cached.size()) : -1;
}

kv_status_t kv_pc_free_queue(const kv_prefix_cache_t* pc, int32_t* blocks, int32_t cap, int32_t* num) {
    if (!pc || !num) return KV_ERR_INVALID_ARG;
    if (pc->num_free > 0 && (!blocks || cap < pc->num_free)) return KV_ERR_INVALID_ARG;
    int32_t i = 0;
    for (int32_t b = pc->head; b >= 0; b = pc->next[b]) blocks[i++] = b;
    *num = i;
    return KV_OK;
}

kv_status_t kv_pc_block_info(const kv_prefix_cache_t* pc, int32_t block, int32_t* ref_count,
                             int32_t* is_cached, uint64_t* hash) {
    if (!pc || block < 0 || block >= pc->num_blocks) return KV_ERR_INVALID_ARG;
    if (ref_count) *ref_count = pc->ref[block];
    if (is_cached) *is_cached = pc->hashed[block];
    if (hash) *hash = pc->hashed[block] ? pc->hash[block] : 0;
    return KV_OK;
}

uint64_t kv_pc_hash_block(uint64_t prev, const int32_t* tokens, int32_t n, int32_t first,
                          uint64_t salt) {
    if (n < 0 || (n > 0 && !tokens)) return 0;
    return chain_hash(prev, tokens, n, first != 0, salt);
}

}  // extern "C"
