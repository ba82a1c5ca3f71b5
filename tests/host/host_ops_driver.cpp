// Host-side driver for the library's block manager and prefix cache, built with the
// address and undefined-behaviour sanitizers by tests/test_host_sanitizers.py (CPU only,
// no GPU code involved).  It runs long random sequences of valid calls, checks the
// managers' invariants after each, and makes invalid calls (unknown ids, null or short
// buffers, out-of-range blocks) that must return an error status and change nothing.
// Prints "ok" and exits 0 on success; any sanitizer report aborts the process.

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <random>
#include <set>
#include <vector>

#include "pagedkv.h"

#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__);     \
            exit(2);                                                             \
        }                                                                        \
    } while (0)

static std::vector<int32_t> free_list(kv_block_manager_t* m, int nb) {
    std::vector<int32_t> v(nb);
    int32_t n = 0;
    CHECK(kv_bm_free_list(m, v.data(), nb, &n) == KV_OK);
    v.resize(n);
    return v;
}

// every block is either free (count 0, listed once) or counted by the tables naming it
static void bm_invariants(kv_block_manager_t* m, int nb, const std::set<int64_t>& live) {
    std::vector<int> refs(nb, 0);
    for (int64_t r : live) {
        int32_t len = 0, n = 0;
        CHECK(kv_bm_get_length(m, r, &len) == KV_OK);
        std::vector<int32_t> t(nb + 1);
        CHECK(kv_bm_get_table(m, r, t.data(), nb + 1, &n) == KV_OK);
        CHECK(n == 0 ? len == 0 : true);
        for (int i = 0; i < n; ++i) {
            CHECK(t[i] >= 0 && t[i] < nb);
            ++refs[t[i]];
        }
    }
    std::vector<int32_t> fl = free_list(m, nb);
    std::vector<int> listed(nb, 0);
    for (int32_t b : fl) ++listed[b];
    for (int b = 0; b < nb; ++b) {
        int32_t c = -1;
        CHECK(kv_bm_ref_count(m, b, &c) == KV_OK);
        CHECK(c == refs[b]);
        CHECK(listed[b] == (refs[b] == 0 ? 1 : 0));
    }
}

static void block_manager_trace(uint32_t seed) {
    std::mt19937 rng(seed);
    const int B = 1 + rng() % 16;
    const int nd = 8 + rng() % 40, nh = 8 + rng() % 40;
    kv_block_manager_t *dev = nullptr, *host = nullptr;
    CHECK(kv_bm_create(nd, B, &dev) == KV_OK && kv_bm_create(nh, B, &host) == KV_OK);
    std::set<int64_t> on_dev, on_host;
    int64_t next = 0;
    for (int step = 0; step < 2000; ++step) {
        const int op = rng() % 7;
        if (op == 0) {
            CHECK(kv_bm_add_request(dev, next) == KV_OK);
            on_dev.insert(next++);
        } else if (op <= 2 && !on_dev.empty()) {
            std::vector<int64_t> rids(on_dev.begin(), on_dev.end());
            std::shuffle(rids.begin(), rids.end(), rng);
            rids.resize(1 + rng() % rids.size());
            std::vector<int32_t> counts(rids.size());
            int64_t total = 0;
            for (auto& c : counts) total += (c = rng() % (2 * B + 1));
            std::vector<int64_t> slots(std::max<int64_t>(total, 1));
            std::vector<int32_t> copies(3 * rids.size());
            int32_t nc = 0;
            const kv_status_t st = kv_bm_append(dev, rids.data(), counts.data(), (int32_t)rids.size(),
                                                slots.data(), total, copies.data(), (int32_t)rids.size(), &nc);
            CHECK(st == KV_OK || st == KV_ERR_OUT_OF_BLOCKS);
            if (st == KV_OK)
                for (int64_t i = 0; i < total; ++i) CHECK(slots[i] >= 0 && slots[i] < (int64_t)nd * B);
        } else if (op == 3 && !on_dev.empty()) {
            const int64_t p = *std::next(on_dev.begin(), rng() % on_dev.size());
            CHECK(kv_bm_fork(dev, p, next) == KV_OK);
            on_dev.insert(next++);
        } else if (op == 4 && !(on_dev.empty() && on_host.empty())) {
            const bool d = on_host.empty() || (!on_dev.empty() && rng() % 2);
            auto& set = d ? on_dev : on_host;
            const int64_t r = *std::next(set.begin(), rng() % set.size());
            CHECK(kv_bm_free_request(d ? dev : host, r) == KV_OK);
            set.erase(r);
        } else if (op >= 5) {
            const bool out = op == 5;
            auto& src = out ? on_dev : on_host;
            auto& dst = out ? on_host : on_dev;
            if (src.empty()) continue;
            std::vector<int64_t> rids;
            for (int64_t r : src)
                if (rng() % 3 == 0) rids.push_back(r);
            if (rids.empty()) rids.push_back(*src.begin());
            const int cap = (out ? nd : nh) * 4 + 4;
            std::vector<int32_t> pairs(2 * cap);
            int32_t np = 0;
            const kv_status_t st = kv_bm_move(out ? dev : host, out ? host : dev, rids.data(),
                                              (int32_t)rids.size(), pairs.data(), cap, &np);
            CHECK(st == KV_OK || st == KV_ERR_OUT_OF_BLOCKS || st == KV_ERR_INVALID_ARG);
            if (st == KV_OK)
                for (int64_t r : rids) {
                    src.erase(r);
                    dst.insert(r);
                }
        }
        bm_invariants(dev, nd, on_dev);
        bm_invariants(host, nh, on_host);
    }
    // invalid calls: errors, no change
    int32_t n = 0, c = 0;
    int64_t bad = -12345;
    CHECK(kv_bm_free_request(dev, bad) == KV_ERR_INVALID_ARG);
    CHECK(kv_bm_fork(dev, bad, next) == KV_ERR_INVALID_ARG);
    CHECK(kv_bm_ref_count(dev, nd, &c) == KV_ERR_INVALID_ARG);
    CHECK(kv_bm_ref_count(dev, -1, &c) == KV_ERR_INVALID_ARG);
    CHECK(kv_bm_get_table(dev, bad, nullptr, 0, &n) == KV_ERR_INVALID_ARG);
    CHECK(kv_bm_append(dev, &bad, nullptr, 1, nullptr, 0, nullptr, 0, &n) != KV_OK);
    CHECK(kv_bm_move(dev, dev, &bad, 1, nullptr, 0, &n) == KV_ERR_INVALID_ARG);
    CHECK(kv_bm_create(0, B, &host) == KV_ERR_INVALID_ARG);
    bm_invariants(dev, nd, on_dev);
    CHECK(kv_bm_destroy(dev) == KV_OK && kv_bm_destroy(host) == KV_OK);
}

static void prefix_cache_trace(uint32_t seed) {
    std::mt19937 rng(seed);
    const int B = 1 + rng() % 16;
    const int nb = 8 + rng() % 64;
    kv_prefix_cache_t* pc = nullptr;
    CHECK(kv_pc_create(nb, B, &pc) == KV_OK);
    std::vector<std::vector<int32_t>> stems(4);
    for (auto& s : stems) {
        s.resize(rng() % (5 * B));
        for (auto& t : s) t = rng() % 20;
    }
    std::set<int64_t> live;
    int64_t next = 0;
    for (int step = 0; step < 2000; ++step) {
        const int op = rng() % 5;
        if (op == 4 && !live.empty()) {       // a decode step over a subset (and a bad one)
            std::vector<int64_t> rids;
            for (int64_t r : live)
                if (rng() % 2) rids.push_back(r);
            std::vector<int32_t> toks(rids.size());
            for (auto& t : toks) t = rng() % 20;
            std::vector<int64_t> slots(rids.size() + 1);
            const kv_status_t st = kv_pc_append_step(pc, rids.empty() ? nullptr : rids.data(),
                                                     toks.empty() ? nullptr : toks.data(),
                                                     (int32_t)rids.size(), slots.data());
            CHECK(st == KV_OK || st == KV_ERR_OUT_OF_BLOCKS);
            if (st == KV_OK)
                for (size_t i = 0; i < rids.size(); ++i) CHECK(slots[i] >= 0 && slots[i] < (int64_t)nb * B);
            if (!rids.empty()) {
                rids.push_back(rids[0]);          // repeated id: rejected, nothing changes
                toks.push_back(0);
                CHECK(kv_pc_append_step(pc, rids.data(), toks.data(), (int32_t)rids.size(),
                                        slots.data()) == KV_ERR_INVALID_ARG);
            }
        } else if (op == 0) {
            std::vector<int32_t> prompt = stems[rng() % stems.size()];
            const int extra = rng() % (2 * B);
            for (int i = 0; i < extra; ++i) prompt.push_back(rng() % 20);
            int32_t found = -1;
            CHECK(kv_pc_add_request(pc, next, prompt.empty() ? nullptr : prompt.data(),
                                    (int32_t)prompt.size(), rng() % 2, &found) == KV_OK);
            CHECK(found >= 0 && found % B == 0 && found <= (int32_t)prompt.size());
            live.insert(next++);
        } else if (op <= 2 && !live.empty()) {
            const int64_t r = *std::next(live.begin(), rng() % live.size());
            std::vector<int32_t> toks(1 + rng() % (3 * B));
            for (auto& t : toks) t = rng() % 20;
            std::vector<int64_t> slots(toks.size());
            const kv_status_t st = kv_pc_append(pc, r, toks.data(), (int32_t)toks.size(), slots.data(),
                                                (int64_t)slots.size());
            CHECK(st == KV_OK || st == KV_ERR_OUT_OF_BLOCKS);
            if (st == KV_OK)
                for (int64_t s : slots) CHECK(s >= 0 && s < (int64_t)nb * B);
        } else if (op == 3 && !live.empty()) {
            const int64_t r = *std::next(live.begin(), rng() % live.size());
            CHECK(kv_pc_free_request(pc, r) == KV_OK);
            live.erase(r);
        }
        // free queue: distinct blocks with no references
        std::vector<int32_t> q(nb);
        int32_t n = 0;
        CHECK(kv_pc_free_queue(pc, q.data(), nb, &n) == KV_OK);
        CHECK(n == kv_pc_num_free(pc));
        std::vector<int> seen(nb, 0);
        for (int i = 0; i < n; ++i) {
            CHECK(q[i] >= 0 && q[i] < nb && !seen[q[i]]);
            seen[q[i]] = 1;
            int32_t ref = -1, cached = -1;
            uint64_t h = 0;
            CHECK(kv_pc_block_info(pc, q[i], &ref, &cached, &h) == KV_OK);
            CHECK(ref == 0);
        }
    }
    int32_t n = 0, ref = 0, cached = 0;
    uint64_t h = 0;
    CHECK(kv_pc_free_request(pc, -7) == KV_ERR_INVALID_ARG);
    CHECK(kv_pc_block_info(pc, nb, &ref, &cached, &h) == KV_ERR_INVALID_ARG);
    CHECK(kv_pc_free_queue(pc, nullptr, 0, &n) != KV_OK || kv_pc_num_free(pc) == 0);
    CHECK(kv_pc_destroy(pc) == KV_OK);
}

int main() {
    for (uint32_t seed = 1; seed <= 12; ++seed) {
        block_manager_trace(seed);
        prefix_cache_trace(seed);
    }
    printf("ok\n");
    return 0;
}
