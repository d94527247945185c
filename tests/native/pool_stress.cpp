// Multithreaded stress of the host page pool (include/kvpool.h), built with
// AddressSanitizer + UndefinedBehaviorSanitizer and, separately, with
// ThreadSanitizer by tests/test_sanitizers.py. Eight threads allocate and free
// pages of one pool at random while a shared ownership map checks that no
// page is ever handed to two owners, that every freed page's tag has moved
// on from the tag its owner recorded, and that the pool's statistics add up.
// Error paths (repeated ids, foreign ids, exhaustion, bad arguments) are
// exercised from the same threads. Prints "ok" and exits 0 on success.
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <thread>
#include <vector>

#include "kvpool.h"

namespace {

constexpr int kPages = 4096;
constexpr int kThreads = 8;
constexpr int kIters = 4000;

std::atomic<int> g_owner[kPages];          // -1 free, else the owning thread
std::atomic<int> g_fail{0};

void fail(const char* what, long a = 0, long b = 0) {
    if (g_fail.fetch_add(1) < 10) std::fprintf(stderr, "FAIL: %s (%ld, %ld)\n", what, a, b);
}

void worker(kv_pool* pool, int t, std::atomic<int64_t>* checks) {
    std::mt19937 rng(1234u + static_cast<unsigned>(t));
    std::vector<int32_t> mine;
    std::vector<uint32_t> my_tags;
    for (int it = 0; it < kIters; ++it) {
        const int op = static_cast<int>(rng() % 10);
        if (op < 5) {                                            // allocate 1..32 pages
            const int n = 1 + static_cast<int>(rng() % 32);
            std::vector<int32_t> pages(n);
            std::vector<uint32_t> tags(n);
            const int st = kv_pool_alloc(pool, n, pages.data(), tags.data());
            if (st == KV_ERR_EXHAUSTED) continue;
            if (st != KV_OK) { fail("alloc status", st); continue; }
            for (int i = 0; i < n; ++i) {
                if (pages[i] < 0 || pages[i] >= kPages) { fail("alloc id", pages[i]); continue; }
                int expect = -1;
                if (!g_owner[pages[i]].compare_exchange_strong(expect, t))
                    fail("page handed out twice", pages[i], expect);
                mine.push_back(pages[i]);
                my_tags.push_back(tags[i]);
            }
        } else if (op < 9 && !mine.empty()) {                   // free some of mine
            const size_t n = 1 + rng() % mine.size();
            std::vector<int32_t> pages(mine.end() - static_cast<long>(n), mine.end());
            std::vector<uint32_t> tags(my_tags.end() - static_cast<long>(n), my_tags.end());
            for (int32_t p : pages) g_owner[p].store(-1);
            const int st = kv_pool_free(pool, pages.data(), static_cast<int32_t>(n));
            if (st != KV_OK) fail("free status", st);
            mine.resize(mine.size() - n);
            my_tags.resize(my_tags.size() - n);
            // a page freed by me: its current tag differs from the one I recorded
            std::vector<uint32_t> now(kPages);
            if (kv_pool_tags(pool, now.data()) != KV_OK) fail("tags");
            for (size_t i = 0; i < n; ++i)
                if (now[pages[i]] == tags[i] && g_owner[pages[i]].load() == -1)
                    fail("tag unchanged after free", pages[i]);
            // a page listed twice is refused, and nothing is freed
            if (!mine.empty()) {
                const int32_t twice[2] = {mine.back(), mine.back()};
                if (kv_pool_free(pool, twice, 2) != KV_ERR_STATE) fail("repeated id accepted");
            }
        } else {                                                  // a tag check outcome
            uint8_t abort[16];
            int bad = 0;
            for (int i = 0; i < 16; ++i) bad += (abort[i] = static_cast<uint8_t>(rng() % 7 == 0));
            if (kv_pool_record_check(pool, abort, 16) != KV_OK) fail("record_check");
            checks[0] += 16;
            checks[1] += bad;
        }
        // bad arguments are refused without side effects
        if (kv_pool_alloc(pool, -1, nullptr, nullptr) != KV_ERR_SHAPE) fail("alloc -1");
        const int32_t foreign = -3;
        if (kv_pool_free(pool, &foreign, 1) != KV_ERR_STATE) fail("free foreign");
    }
    for (int32_t p : mine) g_owner[p].store(-1);
    if (!mine.empty() && kv_pool_free(pool, mine.data(), static_cast<int32_t>(mine.size())) != KV_OK)
        fail("final free");
}

}  // namespace

int main() {
    for (auto& o : g_owner) o.store(-1);
    kv_pool* pool = nullptr;
    if (kv_pool_create(kPages, 1, 99u, &pool) != KV_OK || !pool) return 2;
    std::atomic<int64_t> checks[2];
    checks[0] = 0;
    checks[1] = 0;
    std::vector<std::thread> ts;
    for (int t = 0; t < kThreads; ++t) ts.emplace_back(worker, pool, t, checks);
    for (auto& th : ts) th.join();
    kv_pool_stats s{};
    if (kv_pool_get_stats(pool, &s) != KV_OK) fail("stats");
    if (s.free_pages != kPages) fail("free pages at the end", s.free_pages);
    if (s.pages_allocated != s.pages_freed) fail("allocated != freed", s.pages_allocated, s.pages_freed);
    if (s.requests_checked != checks[0].load()) fail("requests_checked", s.requests_checked);
    if (s.requests_aborted != checks[1].load()) fail("requests_aborted", s.requests_aborted);
    kv_pool_destroy(pool);
    // the no-op tracker: tags stay 0, checks count nothing
    if (kv_pool_create(64, 0, 7u, &pool) != KV_OK) return 2;
    int32_t pages[64];
    uint32_t tags[64];
    if (kv_pool_alloc(pool, 64, pages, tags) != KV_OK) fail("noop alloc");
    if (kv_pool_free(pool, pages, 64) != KV_OK) fail("noop free");
    uint32_t now[64];
    kv_pool_tags(pool, now);
    for (int i = 0; i < 64; ++i)
        if (now[i] != 0u || tags[i] != 0u) fail("noop tag", i);
    kv_pool_destroy(pool);
    kv_pool_destroy(nullptr);
    if (g_fail.load() != 0) return 1;
    std::printf("ok\n");
    return 0;
}
