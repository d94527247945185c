/*
 * kvfp8.h -- C ABI of a paged FP8-e4m3 KV-cache decode library for AMD
 * MI355X (gfx950 / CDNA4).
 *
 * The operations follow the problem statement of the five web reports of
 * Cloudflare's post on serving Kimi and GLM (remio.ai it/pt/ko pages titled
 * "Il serving di modelli più piccoli di Cloudflare riduce la memoria, ma la
 * sicurezza diventa la prova decisiva" and translations; iitog.ru "Cloudflare
 * ускорила Kimi на 41% сжатием KV-кеша ..."; manulx.blog "CloudflareのKimiと
 * GLMを提供するためのレシピ ..."):
 *
 *   - the KV cache is stored in FP8 e4m3 instead of BF16, halving its size
 *     (remio.ai/it, section "Cosa ha cambiato Cloudflare per Kimi e GLM");
 *   - the attention kernel converts the cached values when it reads them
 *     (section "Perché le cache più piccole di Cloudflare battono la velocità
 *     pura");
 *   - every physical cache page carries a tag that changes whenever the page
 *     is reallocated; the server records the pages and tags each request
 *     expects, and before supported decode operations read those pages the
 *     mappings are verified, a mismatch aborting the affected request; the
 *     check is a separate batched operation, not fused into attention, and a
 *     no-op tracker exists where the check is disabled (sections "Cosa ha
 *     cambiato ..." and "La sicurezza della cache KV condivisa diventa una
 *     questione di produzione"; iitog.ru, paragraph on tags; manulx.blog,
 *     "共有キャッシュの保護").
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers, allocated and owned by the
 *     caller. The library allocates nothing, keeps no handles and no state
 *     beyond one exception (paged_decode_attn_append_noalloc's static device
 *     scratch, one per GPU for the life of the process, and its address
 *     cached per device), and is safe to call from several host threads.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously on it; nothing synchronises the host.
 *   - Arguments are validated before anything is enqueued. On invalid
 *     arguments a negative kv_status is returned and nothing is launched.
 *     KV_ERR_LAUNCH reports a HIP launch error seen right after enqueueing.
 *   - Data-plane outcomes are never errors: a tag mismatch or a bad page id
 *     only raises a request's abort flag / zeroes its output. The kernels
 *     never touch memory outside [0, num_pages) pages, whatever the tables
 *     hold.
 *   - Supported shapes: head_dim == 128, page_size == 16, num_q_heads a
 *     multiple of num_kv_heads with group size num_q_heads/num_kv_heads in
 *     [1, 16]. bf16 / FP8 arrays must be 16-byte aligned, int32/uint32/float
 *     arrays 4-byte aligned.
 *
 * Number format. FP8 codes are OCP 8-bit floating point E4M3 ("e4m3fn"):
 * sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, NaN =
 * S.1111.111, largest finite 448. Stored code = round-to-nearest-even of
 * x / s with saturation to +-448 (+-inf included), NaN -> 0x7F/0xFF keeping
 * the sign, and the sign kept on zero, where x / s is the EXACT quotient
 * (the kernels round it to fp32 with round-to-odd first, from the correctly
 * rounded quotient and its exact fma remainder, so the second rounding cannot
 * be misled by a quotient that lands on an e4m3 midpoint). The value read
 * back is code * s. s is one fp32 scale per (layer, KV head) for
 * K and one for V, supplied by the caller (positive and finite).
 *
 * Pool layout. Each layer has a K pool and a V pool, each an array of
 * [num_pages][num_kv_heads] tiles; a tile holds page_size (16) tokens x
 * head_dim (128) elements of one KV head: 2048 bytes for FP8, 4096 bytes for
 * BF16. Tile (page p, head g) starts at byte (p * num_kv_heads + g) * tile.
 * Inside a tile the element of token t (0..15) and dimension d (0..127) is at
 * byte offset
 *
 *   FP8  K: 1024*((d%32)/16) + 256*(d/32) + 16*t + (d%16)
 *   FP8  V: 1024*(d/64) + 256*(t/4) + 16*(d%16) + 4*((d/16)%4) + (t%4)
 *   BF16 K: 1024*((d%32)/8)  + 256*(d/32) + 16*t + 2*(d%8)
 *   BF16 V: 1024*(d/32) + 256*(t/4) + 16*(d%16) + 8*((d/16)%2) + 2*(t%4)
 *
 * (integer division). These are permutations of the tile chosen so that a
 * wavefront reads a tile with fully contiguous 16-byte-per-lane loads that
 * land directly in the register layout of the gfx950 16x16x32 matrix-core
 * instructions: K rows feed the QK^T product, V is stored token-minor so the
 * P.V product needs no transpose. Pools should be written only through the
 * append entry points.
 *
 * Request tables (shared by all layers):
 *   block_table   int32 [batch][bt_stride]  logical page j -> physical page id
 *   expected_tags uint32[batch][bt_stride]  tag the request recorded for page j
 *   pool_tags     uint32[num_pages]         current tag of each physical page
 *   seq_lens      int32 [batch]             tokens attended, INCLUDING the token
 *                                           appended this step
 * Token t of request b lives in page block_table[b][t/16], slot t%16. Only
 * entries j < ceil(seq_lens[b]/16) are ever read.
 */
#ifndef KVFP8_H
#define KVFP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KV_OK = 0,
    KV_ERR_NULL = -1,        /* a required pointer is NULL                          */
    KV_ERR_SHAPE = -2,       /* a size is negative or inconsistent, or so large that
                                one launch would exceed 2^32 - 1 work-items        */
    KV_ERR_UNSUPPORTED = -3, /* head_dim/page_size/group size/partition not handled */
    KV_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than required             */
    KV_ERR_LAUNCH = -5,      /* HIP reported an error when enqueueing               */
    KV_ERR_ALIGN = -6,       /* a pointer is not aligned as required                */
    KV_ERR_EXHAUSTED = -7,   /* page pool: fewer free pages than requested          */
    KV_ERR_STATE = -8        /* page pool: freeing a page that is not allocated     */
} kv_status;

typedef enum { KV_CACHE_FP8_E4M3 = 0, KV_CACHE_BF16 = 1 } kv_cache_dtype;

#define KV_PAGE_SIZE 16
#define KV_HEAD_DIM 128
#define KV_MAX_GROUP 16
#define KV_MAX_PARTITION_TOKENS 16384
#define KV_MAX_PARTITIONS 8192        /* ceil(max_seq_len / partition_tokens) */

/*
 * Batched page-tag check: the separate batch operation that compares each
 * request's recorded (page, tag) pairs with the pool before supported decode
 * operations read, and aborts only the mismatching request (remio.ai/it,
 * sections "Cosa ha cambiato Cloudflare per Kimi e GLM" and "La sicurezza
 * della cache KV condivisa diventa una questione di produzione").
 *
 * For every request b < batch writes abort_out[b] = 1 if
 *   seq_lens[b] < 0, or ceil(seq_lens[b]/page_size) > bt_stride, or
 *   some j < ceil(seq_lens[b]/page_size) has block_table[b][j] outside
 *   [0, num_pages) or pool_tags[block_table[b][j]] != expected_tags[b][j];
 * else abort_out[b] = 0. abort_out is overwritten, never accumulated.
 * Run it before the append and attention calls of the step, on the same
 * stream, and pass abort_out to them. Skipping it and passing abort = NULL to
 * the other calls is the no-op tracker.
 *
 * pool_tags [num_pages], block_table/expected_tags [batch][bt_stride],
 * seq_lens [batch]: read. abort_out uint8 [batch]: written.
 * workspace: optional device memory of kv_verify_tags_workspace_bytes(batch,
 * bt_stride) bytes, zero-filled before its first use; every call leaves it
 * zeroed again. With it, rows of more than KV_VERIFY_CHUNK_PAGES pages are
 * checked by several workgroups whose verdicts the last one combines; with
 * NULL (or when that size is 0) one workgroup checks each whole row. Calls
 * that overlap in time must not share a workspace.
 * Errors: KV_ERR_NULL (any pointer NULL while batch > 0), KV_ERR_SHAPE
 * (batch, num_pages or bt_stride negative, or batch > 4,194,303; with a
 * workspace, batch x ceil(bt_stride / KV_VERIFY_CHUNK_PAGES) > 16,777,215),
 * KV_ERR_UNSUPPORTED (page_size != 16), KV_ERR_WORKSPACE (workspace_bytes
 * below the size above), KV_ERR_ALIGN. batch == 0 enqueues nothing.
 */
#define KV_VERIFY_CHUNK_PAGES 2048
size_t kv_verify_tags_workspace_bytes(int32_t batch, int32_t bt_stride);
int kv_verify_tags(const uint32_t* pool_tags, int32_t num_pages,
                   const int32_t* block_table, const uint32_t* expected_tags,
                   int32_t bt_stride, const int32_t* seq_lens, int32_t batch,
                   int32_t page_size, uint8_t* abort_out, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * Quantize-on-append into an FP8 e4m3 pool: the cache holds e4m3 codes
 * instead of BF16 values (remio.ai/it, section "Cosa ha cambiato Cloudflare
 * per Kimi e GLM"), written through one fp32 scale per (layer, KV head).
 *
 * For each new token n < n_tok, request b = tok_seq[n], position t =
 * tok_pos[n]: if 0 <= b < batch, abort (if non-NULL) has abort[b] == 0,
 * 0 <= t, t/16 < bt_stride and page = block_table[b][t/16] is in
 * [0, num_pages), then for every KV head g and dimension d
 *     K tile (page, g)[t%16][d] = E4M3(k_new[n][g][d] / k_scale[g])
 *     V tile (page, g)[t%16][d] = E4M3(v_new[n][g][d] / v_scale[g])
 * and otherwise nothing is written. Decode appends one token per request
 * (tok_seq = 0..batch-1, tok_pos = seq_lens - 1); bulk mode (prefill
 * ingest) passes any number of (request, position) pairs, distinct targets.
 *
 * k_new, v_new: bf16 [n_tok][num_kv_heads][head_dim], read.
 * k_scale, v_scale: fp32 [num_kv_heads] of this layer, read.
 * k_pool, v_pool: this layer's FP8 pools (layout above), written at targets.
 * Errors: KV_ERR_NULL, KV_ERR_SHAPE (also n_tok > 16,777,215),
 * KV_ERR_UNSUPPORTED (head_dim != 128, page_size != 16), KV_ERR_ALIGN.
 * n_tok == 0 enqueues nothing.
 */
int kv_append_quant(const void* k_new, const void* v_new,
                    const int32_t* tok_seq, const int32_t* tok_pos, int32_t n_tok,
                    const int32_t* block_table, int32_t bt_stride, int32_t batch,
                    const float* k_scale, const float* v_scale,
                    uint8_t* k_pool, uint8_t* v_pool, int32_t num_pages,
                    int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                    const uint8_t* abort, void* stream);

/*
 * BF16-cache append: same addressing and skipping rules as kv_append_quant,
 * the bf16 value stored unchanged (the comparison format kept where compute
 * dominates, remio.ai/it section "Cosa ha cambiato ...").
 */
int kv_append_bf16(const void* k_new, const void* v_new,
                   const int32_t* tok_seq, const int32_t* tok_pos, int32_t n_tok,
                   const int32_t* block_table, int32_t bt_stride, int32_t batch,
                   void* k_pool, void* v_pool, int32_t num_pages,
                   int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                   const uint8_t* abort, void* stream);

/*
 * Split-K partition size (tokens) that paged_decode_attn will use for these
 * sizes and cache_dtype (KV_CACHE_*; anything else: KV_ERR_UNSUPPORTED).
 * partition_tokens > 0 is returned unchanged if it is a multiple of 16 and
 * at most KV_MAX_PARTITION_TOKENS, else KV_ERR_UNSUPPORTED;
 * partition_tokens == 0 picks one (a pure function of the arguments; the
 * BF16 cache, with twice the bytes per token, may get shorter partitions).
 */
int32_t paged_decode_attn_partition_tokens(int32_t batch, int32_t num_kv_heads,
                                           int32_t max_seq_len, int32_t partition_tokens,
                                           int32_t cache_dtype);

/*
 * Bytes of device workspace paged_decode_attn needs for these sizes (0 when a
 * single partition covers max_seq_len). The workspace holds the split-K
 * softmax partials (running max, normaliser, unnormalised output), one slot
 * per partition of each (request, query head) plus one more, that the
 * cross-partition reduction combines. Every call writes the slots it reads,
 * so the contents on entry do not matter and one buffer serves any later
 * calls and sizes that fit it. The partition count, and so the size, depends
 * on cache_dtype when partition_tokens is 0. Returns 0 for unsupported
 * arguments.
 */
size_t paged_decode_attn_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t max_seq_len, int32_t partition_tokens,
                                         int32_t cache_dtype);

/*
 * Decode-step attention over the paged cache, dequantizing on read: the
 * kernel converts the cached codes as it reads them (remio.ai/it, section
 * "Perché le cache più piccole di Cloudflare battono la velocità pura").
 *
 * For each request b with abort[b] == 0 (or abort == NULL) and
 * 1 <= L = seq_lens[b] <= max_seq_len whose pages j < ceil(L/16) are all
 * valid ids, and each query head h with KV head g = h / (Hq/Hkv):
 *     K_j = code_K(token j, g) * k_scale[g],  V_j likewise with v_scale
 *          (BF16 cache: the stored bf16 values, scales ignored)
 *     s_j = sm_scale * (q[b][h] . K_j),  p = softmax_j(s),
 *     out[b][h][:] = sum_j p_j V_j
 * and out[b][h][:] = 0 for every other request (aborted, empty, too long,
 * or mapped to an invalid page). The sequence is split into partitions of
 * partition_tokens tokens (0 = automatic); each is reduced with an online
 * softmax, and with more than one partition a second kernel merges the
 * partials.
 *
 * sm_scale must be finite and >= 0 (usually 1/sqrt(head_dim)); the scales
 * must be positive and finite.
 * q: bf16 [batch][num_q_heads][head_dim]. out: fp32 [batch][num_q_heads]
 * [head_dim], fully written. k_scale/v_scale: fp32 [num_kv_heads] (may be
 * NULL for the BF16 cache). workspace: device memory of at least
 * paged_decode_attn_workspace_bytes(...) bytes (may be NULL when that size
 * is 0).
 * Errors: KV_ERR_NULL, KV_ERR_SHAPE (also when partitions x batch x
 * num_kv_heads exceeds 8,388,607, or, with more than one partition, batch x
 * num_q_heads does), KV_ERR_UNSUPPORTED (also when
 * ceil(max_seq_len / partition_tokens) exceeds KV_MAX_PARTITIONS, or for a
 * negative or non-finite sm_scale),
 * KV_ERR_WORKSPACE, KV_ERR_ALIGN, KV_ERR_LAUNCH.
 */
int paged_decode_attn(const void* q, int32_t cache_dtype,
                      const void* k_pool, const void* v_pool,
                      const float* k_scale, const float* v_scale,
                      const int32_t* block_table, int32_t bt_stride,
                      const int32_t* seq_lens, int32_t max_seq_len,
                      const uint8_t* abort, float* out, float sm_scale,
                      int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t page_size, int32_t num_pages,
                      int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * One decode step's append and attention for one layer in a single launch:
 * the same result as kv_append_quant (FP8) / kv_append_bf16 (BF16) with
 * tok_seq = 0..batch-1, tok_pos = seq_lens - 1, followed by paged_decode_attn,
 * for every request the attention accepts (abort[b] == 0, 1 <= L <= max_seq_len,
 * ceil(L/16) <= bt_stride). The new token is written when its request is
 * accepted and maps only valid pool pages. A request that maps an invalid
 * page gets zeros, and whether its new token is stored is left open (run
 * the tag check first and such a request is aborted: neither written nor
 * read). The wavefront that
 * processes the new token's page quantizes it, uses the codes from its
 * registers and stores them for later steps, so nothing in the launch reads
 * them back from memory. One launch per layer instead of two; the separate
 * calls remain for bulk ingest and for callers that need them apart. The
 * pages define the two operations (quantize on write, convert on read:
 * remio.ai/it, sections "Cosa ha cambiato Cloudflare per Kimi e GLM" and
 * "Perché le cache più piccole di Cloudflare battono la velocità pura");
 * fusing them is this library's choice, and the tag check stays separate.
 *
 * k_new, v_new: bf16 [batch][num_kv_heads][head_dim], read. k_pool, v_pool are
 * written (the new token's slot) and read. Other arguments and errors as for
 * paged_decode_attn (KV_ERR_NULL also for a NULL k_new / v_new).
 */
int paged_decode_attn_append(const void* q, const void* k_new, const void* v_new,
                             int32_t cache_dtype, void* k_pool, void* v_pool,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_table, int32_t bt_stride,
                             const int32_t* seq_lens, int32_t max_seq_len, const uint8_t* abort,
                             float* out, float sm_scale, int32_t batch, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                             int32_t num_pages, int32_t partition_tokens, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * paged_decode_attn_append without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). The split-K workspace is a static
 * device array of KV_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends; the call allocates nothing. Same
 * arguments and result as paged_decode_attn_append otherwise. Sizes whose
 * workspace (paged_decode_attn_workspace_bytes) exceeds the array are refused
 * with KV_ERR_WORKSPACE before anything is enqueued. All calls on one GPU
 * share that GPU's array: calls that may overlap in time on one GPU (other
 * streams, other host threads) race and must not be issued; calls in order on
 * one stream are fine. KV_ERR_LAUNCH also if the array's device address
 * cannot be obtained.
 */
#define KV_NOALLOC_SCRATCH_BYTES (64u << 20)
int paged_decode_attn_append_noalloc(const void* q, const void* k_new, const void* v_new,
                                     int32_t cache_dtype, void* k_pool, void* v_pool,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* block_table, int32_t bt_stride,
                                     const int32_t* seq_lens, int32_t max_seq_len,
                                     const uint8_t* abort, float* out, float sm_scale,
                                     int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t page_size, int32_t num_pages,
                                     int32_t partition_tokens, void* stream);

/*
 * Prefill ingest: the handoff of a prompt's BF16 keys and values into the
 * decode cache. The pages run prefill and decode in separate pools; prefill
 * builds a prompt's initial cache state in BF16, decode reads the smaller
 * FP8 cache (remio.ai/it, sections "Cosa ha cambiato Cloudflare per Kimi e
 * GLM" and "Perché le cache più piccole di Cloudflare battono la velocità
 * pura"). Calibration then ingest, per layer:
 *     kv_amax_accumulate(k rows, ..., amax_k)   (amax_k starts at zeros;
 *     kv_amax_accumulate(v rows, ..., amax_v)    call once per chunk of rows)
 *     kv_scales_from_amax(amax_k, Hkv, k_scale); likewise for V
 *     kv_ingest_prefill(...)
 * The calibration rule (scale = amax / 448 per (layer, KV head)) is this
 * library's reading; the pages state none.
 */

/*
 * amax_inout[g] = max(amax_inout[g], max |x[r][g][d]|) over rows r < n_rows
 * and d < head_dim, taking only finite values (NaN and +-Inf are skipped).
 * x: bf16 [n_rows][num_kv_heads][head_dim], 16-byte aligned. amax_inout: fp32
 * [num_kv_heads], finite and >= 0 on entry (zeros to start), updated with
 * device atomics, so concurrent calls on one array are allowed. The result
 * is exact (a maximum). Errors: KV_ERR_SHAPE, KV_ERR_UNSUPPORTED
 * (head_dim != 128), KV_ERR_NULL, KV_ERR_ALIGN, KV_ERR_LAUNCH.
 */
int kv_amax_accumulate(const void* x, int64_t n_rows, int32_t num_kv_heads, int32_t head_dim,
                       float* amax_inout, void* stream);

/*
 * scale_out[i] = max(fp32(amax[i] / 448), FLT_MIN) (correctly rounded
 * division) for finite amax[i] > 0, else 1.0. Every scale is a positive
 * normal fp32, as kv_append_quant / kv_ingest_prefill require.
 * amax, scale_out: fp32 [n] (may alias). Errors: KV_ERR_SHAPE, KV_ERR_NULL,
 * KV_ERR_ALIGN, KV_ERR_LAUNCH.
 */
int kv_scales_from_amax(const float* amax, int32_t n, float* scale_out, void* stream);

/*
 * Write whole prompts into the pool, page by page. Token t of request b is
 * row row_start[b] + t of k_rows / v_rows (bf16 [n_rows][num_kv_heads]
 * [head_dim]). For every request b with abort[b] == 0 (or abort == NULL),
 * 1 <= L = seq_lens[b] <= max_seq_len, ceil(L/16) <= bt_stride and
 * 0 <= row_start[b], row_start[b] + L <= n_rows, and every page j < ceil(L/16)
 * whose id p = block_table[b][j] is in [0, num_pages), and each KV head g:
 *     tile (p, g) slot s = E4M3(x / scale[g]) of token 16 j + s  (FP8; BF16:
 *                          the bits unchanged), for 16 j + s < L
 *     tile (p, g) slot s = 0 (code or bits) for 16 j + s >= L
 * i.e. the same codes kv_append_quant writes for those tokens, in whole tiles
 * with full 16-byte stores. Other requests and pages are not touched.
 * k_scale, v_scale: fp32 [num_kv_heads], positive normal (FP8; ignored and
 * may be NULL for BF16). cache_dtype selects the pool format. Any batch x
 * ceil(max_seq_len / 16) is accepted (the kernel loops over the pages).
 * Errors: KV_ERR_SHAPE, KV_ERR_UNSUPPORTED, KV_ERR_NULL, KV_ERR_ALIGN,
 * KV_ERR_LAUNCH.
 */
int kv_ingest_prefill(const void* k_rows, const void* v_rows, int64_t n_rows,
                      const int32_t* row_start, const int32_t* seq_lens, int32_t batch,
                      int32_t max_seq_len, const int32_t* block_table, int32_t bt_stride,
                      int32_t cache_dtype, const float* k_scale, const float* v_scale,
                      void* k_pool, void* v_pool, int32_t num_pages, int32_t num_kv_heads,
                      int32_t head_dim, int32_t page_size, const uint8_t* abort, void* stream);

/*
 * Weight-only quantized decode GEMV. The pages compress GLM's weights from
 * FP8 to INT4 for decode, where the weights are streamed from HBM for every
 * token and fewer bytes give each token sooner; the codes are expanded before
 * the product (remio.ai/it, section "La compressione dei pesi GLM modifica il
 * compromesso tra le fasi"). Formats (this library's reading; the pages give
 * only "four-bit integer"): weights W [n][k] in bf16 are quantized per row and
 * per group of 128 inputs with one fp32 scale s:
 *   WQ_INT4:      q = RNE(w / s) of the exact quotient, s = amax / 7, so
 *                 |q| <= 7 (|w / s| <= amax / fp32(amax / 7) < 7.5)
 *   WQ_FP8_E4M3:  q = E4M3(w / s) (the KV encoder), s = amax / 448
 * (s = 1.0 for an all-zero group; weights must be finite), and the product is
 *   y[m][n] += sum_k x[m][k] * q[n][k] * s[n][k / 128]
 * for bf16 activations x [m][k] and fp32 y [m][n].
 *
 * Packed layout (MFMA operand order), block (nt, g) = rows 16 nt .. 16 nt + 15,
 * inputs 128 g .. 128 g + 127, blocks ordered nt-major: block index
 * b = nt * (k / 128) + g. Element (row 16 nt + r, input 128 g + 32 c + 8 j + i),
 * r < 16, c < 4, j < 4, i < 8, with lane l = 16 j + r:
 *   WQ_INT4:     dword 256 b + 4 l + c (bytes 4 x that), sign-magnitude
 *                fields: for i < 4, |q| in bits 0..2 and the sign in bit 7
 *                of byte i % 4; for i >= 4, |q| in bits 4..6 of byte i % 4
 *                and the sign in bit 3 of byte (i + 1) % 4 (bytes of the
 *                dword; zero is always positive);
 *   WQ_FP8_E4M3: byte 2048 b + 1024 (c / 2) + 16 l + 8 (c % 2) + i.
 * Scales: fp32 [n / 16][k / 128][16], element (b, r) = s of row 16 nt + r.
 */
#define WQ_INT4 0
#define WQ_FP8_E4M3 1

/* Bytes of the packed codes for an n x k matrix (0 if n % 16, k % 128 or the
 * format is unsupported). Scales take n * (k / 128) * 4 bytes. */
size_t wq_packed_bytes(int32_t n, int32_t k, int32_t format);

/*
 * Quantize bf16 weights w [n][k] (row-major, device) into packed codes and
 * scales (layouts above). Requires n % 16 == 0, k % 128 == 0. Errors:
 * KV_ERR_SHAPE (also (n / 16) x (k / 128) > 67,108,860), KV_ERR_UNSUPPORTED,
 * KV_ERR_NULL, KV_ERR_ALIGN, KV_ERR_LAUNCH.
 */
int wq_quantize_pack(const void* w, int32_t n, int32_t k, int32_t format, void* packed,
                     float* scales, void* stream);

/*
 * y[m][n] += x[m][:] . dequant(W)[n][:] for m rows of bf16 activations x
 * [m][k] and packed weights (any m; 64 rows per launch). y must hold zeros or
 * a bias on entry: partial sums over ranges of inputs are added with fp32
 * atomics, so the last bits of y may differ between runs. All pointers
 * 16-byte aligned. Errors: KV_ERR_SHAPE (also ceil(n / 64) x (k / 128) >
 * 16,777,215), KV_ERR_UNSUPPORTED, KV_ERR_NULL, KV_ERR_ALIGN, KV_ERR_LAUNCH.
 */
int wq_gemv(const void* x, int32_t m, const void* packed, const float* scales, int32_t n,
            int32_t k, int32_t format, float* y, void* stream);

/* Human-readable name of a kv_status value (static string, never NULL). */
const char* kv_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVFP8_H */
