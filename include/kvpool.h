/*
 * kvpool.h -- host-side page pool and tag tracker for the paged KV cache
 * (part of libkvfp8.so; plain host C++, no GPU calls).
 *
 * The pages this follows (remio.ai/it "Il serving di modelli più piccoli di
 * Cloudflare riduce la memoria, ma la sicurezza diventa la prova decisiva",
 * sections "Cosa ha cambiato Cloudflare per Kimi e GLM" and "La sicurezza
 * della cache KV condivisa diventa una questione di produzione"; iitog.ru and
 * manulx.blog, cache-protection paragraphs) describe the bookkeeping that
 * feeds the batched tag check: every physical page carries a tag that
 * changes whenever the page is reallocated; the server records, for each
 * request, the pages and tags it expects; a mismatch aborts only that request;
 * a no-op tracker exists where the check is disabled; and the mismatch rate
 * is something to monitor. This pool is that state machine:
 *
 *   - kv_pool_alloc hands out free pages with their current tags (what the
 *     request records as its expected tags, next to the page ids in its
 *     block-table row);
 *   - kv_pool_free returns pages and bumps each one's tag (mod 2^32), so any
 *     mapping recorded before the free no longer matches, from the moment of
 *     the free on (a page is therefore reallocated with a new tag);
 *   - kv_pool_tags exports the current tags for the device copy that
 *     kv_verify_tags reads;
 *   - kv_pool_record_check accumulates the outcome of each tag check (the
 *     abort flags copied back to the host) into the mismatch-rate counters.
 *
 * A pool created untracked is the no-op tracker: it allocates and frees
 * pages the same way, every tag is and stays 0, and kv_pool_record_check
 * counts nothing; its callers skip kv_verify_tags and pass abort = NULL.
 *
 * Tracked pools start with tags drawn from a counter-based hash of (seed,
 * page id). The free list is last-in first-out: the most recently freed page
 * is handed out first. All calls are thread-safe (one mutex per pool). Every
 * call validates its arguments first and changes nothing on error; alloc and
 * free are all-or-nothing.
 */
#ifndef KVPOOL_H
#define KVPOOL_H

#include <stdint.h>

#include "kvfp8.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kv_pool kv_pool; /* opaque */

typedef struct {
    int64_t num_pages;
    int64_t free_pages;
    int64_t pages_allocated;     /* pages handed out by kv_pool_alloc, cumulative */
    int64_t pages_freed;         /* pages returned by kv_pool_free, cumulative    */
    int64_t checks;              /* kv_pool_record_check calls (tracked pools)    */
    int64_t requests_checked;    /* requests covered by those checks              */
    int64_t requests_aborted;    /* of which flagged (mismatch or bad mapping)    */
} kv_pool_stats;

/*
 * A pool of num_pages physical pages (ids 0 .. num_pages - 1), all free.
 * tracked != 0 keeps tags (initial values from seed); tracked == 0 is the
 * no-op tracker. *out receives the handle (owned by the caller; release with
 * kv_pool_destroy). Errors: KV_ERR_NULL (out), KV_ERR_SHAPE (num_pages < 0).
 */
int kv_pool_create(int32_t num_pages, int32_t tracked, uint32_t seed, kv_pool** out);

/* Releases the pool (NULL is ignored). */
void kv_pool_destroy(kv_pool* pool);

/*
 * Allocates n pages: pages_out[i] receives a page id, tags_out[i] (may be
 * NULL) its current tag. All or nothing: KV_ERR_EXHAUSTED if fewer than n
 * pages are free. Errors also: KV_ERR_NULL, KV_ERR_SHAPE (n < 0).
 */
int kv_pool_alloc(kv_pool* pool, int32_t n, int32_t* pages_out, uint32_t* tags_out);

/*
 * Frees n pages (each must be allocated, and listed once) and bumps each
 * one's tag by 1 (tracked pools). All or nothing: KV_ERR_STATE if any id is
 * out of range, not allocated, or repeated. Errors also: KV_ERR_NULL,
 * KV_ERR_SHAPE.
 */
int kv_pool_free(kv_pool* pool, const int32_t* pages, int32_t n);

/* Copies the current tag of every page into tags_out[num_pages]. */
int kv_pool_tags(const kv_pool* pool, uint32_t* tags_out);

/*
 * Records one tag check of a batch: abort[batch] are the flags kv_verify_tags
 * produced (copied to the host). Tracked pools add 1 check, batch requests
 * and the number of nonzero flags to the counters; the no-op tracker counts
 * nothing. Errors: KV_ERR_NULL, KV_ERR_SHAPE (batch < 0).
 */
int kv_pool_record_check(kv_pool* pool, const uint8_t* abort, int32_t batch);

/* Copies the counters; the mismatch rate is requests_aborted / requests_checked. */
int kv_pool_get_stats(const kv_pool* pool, kv_pool_stats* out);

#ifdef __cplusplus
}
#endif

#endif /* KVPOOL_H */
