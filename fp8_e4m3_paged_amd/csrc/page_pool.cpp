// Host-side page pool and tag tracker (the bookkeeping that feeds the
// batched tag check; the C ABI and its semantics are in kvpool.h). Plain
// host C++: a LIFO free list, an allocated flag and a 32-bit tag per page,
// the mismatch-rate counters, one mutex.
#include "kvpool.h"

#include <mutex>
#include <new>
#include <vector>

struct kv_pool {
    int32_t num_pages = 0;
    bool tracked = true;
    std::vector<int32_t> free_list;      // top = back(): handed out next
    std::vector<uint8_t> allocated;
    std::vector<uint32_t> tags;
    int64_t pages_allocated = 0;
    int64_t pages_freed = 0;
    int64_t checks = 0;
    int64_t requests_checked = 0;
    int64_t requests_aborted = 0;
    mutable std::mutex mu;
};

namespace {

// MurmurHash3's 32-bit finaliser (Appleby), applied twice to mix (seed, id):
// initial tags only have to be unrelated across pages and pools.
uint32_t fmix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85EBCA6Bu;
    h ^= h >> 13;
    h *= 0xC2B2AE35u;
    h ^= h >> 16;
    return h;
}

}  // namespace

extern "C" {

int kv_pool_create(int32_t num_pages, int32_t tracked, uint32_t seed, kv_pool** out) {
    if (!out) return KV_ERR_NULL;
    if (num_pages < 0) return KV_ERR_SHAPE;
    kv_pool* p = new (std::nothrow) kv_pool();
    if (!p) return KV_ERR_EXHAUSTED;
    p->num_pages = num_pages;
    p->tracked = tracked != 0;
    p->free_list.resize(num_pages);
    // pages are handed out in increasing id order from a fresh pool
    for (int32_t i = 0; i < num_pages; ++i) p->free_list[i] = num_pages - 1 - i;
    p->allocated.assign(num_pages, 0);
    p->tags.assign(num_pages, 0u);
    if (p->tracked)
        for (int32_t i = 0; i < num_pages; ++i)
            p->tags[i] = fmix32(fmix32(static_cast<uint32_t>(i) ^ seed) + 0x9E3779B9u);
    *out = p;
    return KV_OK;
}

void kv_pool_destroy(kv_pool* pool) { delete pool; }

int kv_pool_alloc(kv_pool* pool, int32_t n, int32_t* pages_out, uint32_t* tags_out) {
    if (!pool) return KV_ERR_NULL;
    if (n < 0) return KV_ERR_SHAPE;
    if (n == 0) return KV_OK;
    if (!pages_out) return KV_ERR_NULL;
    std::lock_guard<std::mutex> lock(pool->mu);
    if (static_cast<size_t>(n) > pool->free_list.size()) return KV_ERR_EXHAUSTED;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t id = pool->free_list.back();
        pool->free_list.pop_back();
        pool->allocated[id] = 1;
        pages_out[i] = id;
        if (tags_out) tags_out[i] = pool->tags[id];
    }
    pool->pages_allocated += n;
    return KV_OK;
}

int kv_pool_free(kv_pool* pool, const int32_t* pages, int32_t n) {
    if (!pool) return KV_ERR_NULL;
    if (n < 0) return KV_ERR_SHAPE;
    if (n == 0) return KV_OK;
    if (!pages) return KV_ERR_NULL;
    std::lock_guard<std::mutex> lock(pool->mu);
    // validate everything first (all or nothing): in range, allocated, listed once
    std::vector<uint8_t> seen(pool->num_pages, 0);
    for (int32_t i = 0; i < n; ++i) {
        const int32_t id = pages[i];
        if (id < 0 || id >= pool->num_pages || !pool->allocated[id] || seen[id])
            return KV_ERR_STATE;
        seen[id] = 1;
    }
    for (int32_t i = 0; i < n; ++i) {
        const int32_t id = pages[i];
        pool->allocated[id] = 0;
        if (pool->tracked) pool->tags[id] += 1u;     // stale mappings stop matching now
        pool->free_list.push_back(id);
    }
    pool->pages_freed += n;
    return KV_OK;
}

int kv_pool_tags(const kv_pool* pool, uint32_t* tags_out) {
    if (!pool || (!tags_out && pool->num_pages > 0)) return KV_ERR_NULL;
    std::lock_guard<std::mutex> lock(pool->mu);
    for (int32_t i = 0; i < pool->num_pages; ++i) tags_out[i] = pool->tags[i];
    return KV_OK;
}

int kv_pool_record_check(kv_pool* pool, const uint8_t* abort, int32_t batch) {
    if (!pool) return KV_ERR_NULL;
    if (batch < 0) return KV_ERR_SHAPE;
    if (batch > 0 && !abort) return KV_ERR_NULL;
    std::lock_guard<std::mutex> lock(pool->mu);
    if (!pool->tracked) return KV_OK;
    int64_t bad = 0;
    for (int32_t b = 0; b < batch; ++b) bad += abort[b] != 0;
    pool->checks += 1;
    pool->requests_checked += batch;
    pool->requests_aborted += bad;
    return KV_OK;
}

int kv_pool_get_stats(const kv_pool* pool, kv_pool_stats* out) {
    if (!pool || !out) return KV_ERR_NULL;
    std::lock_guard<std::mutex> lock(pool->mu);
    out->num_pages = pool->num_pages;
    out->free_pages = static_cast<int64_t>(pool->free_list.size());
    out->pages_allocated = pool->pages_allocated;
    out->pages_freed = pool->pages_freed;
    out->checks = pool->checks;
    out->requests_checked = pool->requests_checked;
    out->requests_aborted = pool->requests_aborted;
    return KV_OK;
}

}  // extern "C"
