// C-ABI entry points: argument validation, partition sizing and dispatch to
// the kernel launchers. Validation happens before any HIP call, so invalid
// arguments return a negative status and enqueue nothing.
#include "kvfp8.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kv_launch.h"

namespace {

inline bool misaligned(const void* p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0;
}

inline int launch_status(hipError_t e) { return e == hipSuccess ? KV_OK : KV_ERR_LAUNCH; }

// A launch holds at most 2^32 - 1 work-items; sizes that would need more are
// refused (KV_ERR_SHAPE) before anything is enqueued.
inline bool grid_fits(int64_t workgroups, int64_t threads) {
    return workgroups <= 0xFFFFFFFFLL / threads;
}

int check_append_common(const void* k_new, const void* v_new, const int32_t* tok_seq,
                        const int32_t* tok_pos, int32_t n_tok, const int32_t* block_table,
                        int32_t bt_stride, int32_t batch, const void* k_pool, const void* v_pool,
                        int32_t num_pages, int32_t num_kv_heads, int32_t head_dim,
                        int32_t page_size, const uint8_t* /*abort*/) {
    if (n_tok < 0 || bt_stride < 0 || batch < 0 || num_pages < 0 || num_kv_heads <= 0)
        return KV_ERR_SHAPE;
    if (head_dim != KV_HEAD_DIM || page_size != KV_PAGE_SIZE) return KV_ERR_UNSUPPORTED;
    if (!grid_fits(n_tok, 256)) return KV_ERR_SHAPE;     // one row of workgroups per token
    if (n_tok == 0) return KV_OK;
    if (!k_new || !v_new || !tok_seq || !tok_pos || !block_table || !k_pool || !v_pool)
        return KV_ERR_NULL;
    if (misaligned(k_new, 16) || misaligned(v_new, 16) || misaligned(k_pool, 16) ||
        misaligned(v_pool, 16) || misaligned(tok_seq, 4) || misaligned(tok_pos, 4) ||
        misaligned(block_table, 4))
        return KV_ERR_ALIGN;
    return KV_OK;
}

// Automatic split-K size. Long partitions stream best (the per-workgroup
// set-up and the partial traffic are amortised, and no reduction pass is
// needed with one partition), so split only as far as needed to keep 8
// wavefronts streaming on every compute unit, and into at most 16 partitions
// (the combine then takes one round trip: at one request of 9,193 tokens the
// FP8 step went from 0.129 ms with 18 partitions to 0.107 ms with 12).
// Partitions are equal shares of max_seq_len rounded up to 256 tokens (the
// same number of page pairs for each of 8 wavefronts: at 8 requests 2,304
// tokens ran 3% faster than 2,272), or to one page pair (32 tokens) where the
// coarser rounding would drop partitions; at most the LDS page list's
// capacity, and at least 192 KiB of K and V per KV head (768 FP8 or 384 BF16
// tokens): below that the wavefronts' pipeline start-up dominates. At that
// one request the FP8 step takes 0.107 ms with 12 partitions of 768 tokens
// and 0.125 ms with 16 of 576, while the BF16 step takes 0.143 ms with 16
// and 0.168 ms with 12.
int32_t auto_partition(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len, bool fp8) {
    const int64_t items = static_cast<int64_t>(batch) * num_kv_heads;
    int64_t parts;
    if (items >= 512) parts = 1;
    else if (items <= 256 && 256 % items == 0) parts = 256 / items;
    else parts = (512 + items - 1) / items;
    if (parts > 16) parts = 16;
    const int64_t share = (static_cast<int64_t>(max_seq_len) + parts - 1) / parts;
    int64_t tokens = ((share + 255) / 256) * 256;
    if ((static_cast<int64_t>(max_seq_len) + tokens - 1) / tokens < parts)
        tokens = ((share + 31) / 32) * 32;
    const int64_t min_tokens = (192 * 1024) / (2 * KV_HEAD_DIM * (fp8 ? 1 : 2));
    if (tokens < min_tokens) tokens = min_tokens;
    if (tokens > KV_MAX_PARTITION_TOKENS) tokens = KV_MAX_PARTITION_TOKENS;
    return static_cast<int32_t>(tokens);
}

}  // namespace

// ---- the no-alloc entry point's scratch ------------------------------------
// The split-K workspace of paged_decode_attn_append_noalloc: a static device
// array that every GPU the library runs on holds (zero-filled when the code
// object is loaded) until the process ends. Host code never uses the array's
// name as an address: the first call on a device asks the runtime for that
// device's copy (hipGetSymbolAddress, with that device current) and keeps the
// pointer; kernels receive that pointer. Every call overwrites the partials
// it reads, so no call needs the array cleared. Calls that overlap on one GPU
// share the array and race.
static __device__ __align__(256) uint8_t scratch[KV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The scratch's device address on the device `stream` belongs to (the
// current device for the null stream).
int scratch_for_stream(hipStream_t stream, void** out) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return KV_ERR_LAUNCH;
    int dev = cur;
    if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return KV_ERR_LAUNCH;
    if (dev < 0 || dev >= kMaxDevices) return KV_ERR_LAUNCH;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (dev != cur && hipSetDevice(dev) != hipSuccess) return KV_ERR_LAUNCH;
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (dev != cur && hipSetDevice(cur) != hipSuccess) return KV_ERR_LAUNCH;
            if (e != hipSuccess || p == nullptr) return KV_ERR_LAUNCH;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return KV_OK;
}

}  // namespace

// Shared body of paged_decode_attn (k_new = v_new = NULL: read only) and
// paged_decode_attn_append (the new token is written by the kernel first).
static int attn_impl(const void* q, const void* k_new, const void* v_new, int32_t cache_dtype,
                     void* k_pool, void* v_pool, const float* k_scale, const float* v_scale,
                     const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                     int32_t max_seq_len, const uint8_t* abort, float* out, float sm_scale,
                     int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t page_size, int32_t num_pages, int32_t partition_tokens,
                     void* workspace, size_t workspace_bytes, void* stream,
                     bool static_workspace = false) {
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || bt_stride < 0 || num_pages < 0 ||
        max_seq_len < 0)
        return KV_ERR_SHAPE;
    if (num_q_heads % num_kv_heads != 0) return KV_ERR_SHAPE;
    if (head_dim != KV_HEAD_DIM || page_size != KV_PAGE_SIZE) return KV_ERR_UNSUPPORTED;
    if (num_q_heads / num_kv_heads > KV_MAX_GROUP) return KV_ERR_UNSUPPORTED;
    if (cache_dtype != KV_CACHE_FP8_E4M3 && cache_dtype != KV_CACHE_BF16)
        return KV_ERR_UNSUPPORTED;
    if (!(sm_scale >= 0.0f) || !(sm_scale < INFINITY)) return KV_ERR_UNSUPPORTED;
    const int32_t pt = paged_decode_attn_partition_tokens(batch, num_kv_heads, max_seq_len,
                                                          partition_tokens, cache_dtype);
    if (pt <= 0) return KV_ERR_UNSUPPORTED;
    const int64_t parts64 = max_seq_len == 0 ? 1 : (static_cast<int64_t>(max_seq_len) + pt - 1) / pt;
    if (parts64 > KV_MAX_PARTITIONS) return KV_ERR_UNSUPPORTED;
    // shared-mode grid: one workgroup of up to 8 wavefronts per (partition,
    // request, KV head); the reduce (one wavefront per (request, query head))
    // is held to the same 512 work-items per row
    if (!grid_fits(parts64 * batch * num_kv_heads, 512)) return KV_ERR_SHAPE;
    if (parts64 > 1 && !grid_fits(static_cast<int64_t>(batch) * num_q_heads, 512))
        return KV_ERR_SHAPE;
    if (batch == 0) return KV_OK;
    const bool fp8 = cache_dtype == KV_CACHE_FP8_E4M3;
    if (!q || !out || !seq_lens || !block_table || !k_pool || !v_pool) return KV_ERR_NULL;
    if ((k_new == nullptr) != (v_new == nullptr)) return KV_ERR_NULL;
    if (k_new && (misaligned(k_new, 16) || misaligned(v_new, 16))) return KV_ERR_ALIGN;
    if (fp8 && (!k_scale || !v_scale)) return KV_ERR_NULL;
    if (misaligned(q, 16) || misaligned(out, 16) || misaligned(k_pool, 16) ||
        misaligned(v_pool, 16) || misaligned(seq_lens, 4) || misaligned(block_table, 4) ||
        (k_scale && misaligned(k_scale, 4)) || (v_scale && misaligned(v_scale, 4)))
        return KV_ERR_ALIGN;
    const int32_t parts = static_cast<int32_t>(parts64);
    const size_t need = paged_decode_attn_workspace_bytes(batch, num_q_heads, num_kv_heads,
                                                          head_dim, max_seq_len, pt, cache_dtype);
    if (parts > 1 && static_workspace) {
        // the library's own scratch, resolved only after every check passed
        if (need > KV_NOALLOC_SCRATCH_BYTES) return KV_ERR_WORKSPACE;
        const int r = scratch_for_stream(static_cast<hipStream_t>(stream), &workspace);
        if (r != KV_OK) return r;
        workspace_bytes = KV_NOALLOC_SCRATCH_BYTES;
    }
    if (parts > 1) {
        if (!workspace || workspace_bytes < need) return KV_ERR_WORKSPACE;
        if (misaligned(workspace, 16)) return KV_ERR_ALIGN;
    }
    kvfp8::AttnArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_table = block_table;
    a.bt_stride = bt_stride;
    a.seq_lens = seq_lens;
    a.max_seq_len = max_seq_len;
    a.abort = abort;
    a.out = out;
    a.sm_scale = sm_scale;
    a.batch = batch;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.num_pages = num_pages;
    a.partition_tokens = pt;
    a.num_partitions = parts;
    if (parts > 1) {
        const kvfp8::WorkspaceLayout w = kvfp8::workspace_layout(batch, num_q_heads, parts);
        char* base = static_cast<char*>(workspace);
        a.part_ml = reinterpret_cast<float*>(base + w.ml);
        a.part_acc = reinterpret_cast<float*>(base + w.acc);
    }
    return launch_status(kvfp8::launch_decode_attn(fp8, a, static_cast<hipStream_t>(stream)));
}


extern "C" {

const char* kv_status_str(int status) {
    switch (status) {
        case KV_OK: return "KV_OK";
        case KV_ERR_NULL: return "KV_ERR_NULL: a required pointer is NULL";
        case KV_ERR_SHAPE: return "KV_ERR_SHAPE: a size is negative or inconsistent";
        case KV_ERR_UNSUPPORTED:
            return "KV_ERR_UNSUPPORTED: head_dim/page_size/group size/partition not supported";
        case KV_ERR_WORKSPACE: return "KV_ERR_WORKSPACE: workspace missing or too small";
        case KV_ERR_LAUNCH: return "KV_ERR_LAUNCH: HIP reported an error when enqueueing";
        case KV_ERR_ALIGN: return "KV_ERR_ALIGN: a pointer is not aligned as required";
        case KV_ERR_EXHAUSTED: return "KV_ERR_EXHAUSTED: not enough free pages in the pool";
        case KV_ERR_STATE: return "KV_ERR_STATE: page not allocated (double free or bad id)";
        default: return "unknown kv_status";
    }
}

static_assert(kvfp8::kVerifyChunkPages == KV_VERIFY_CHUNK_PAGES, "tag-check chunk");

size_t kv_verify_tags_workspace_bytes(int32_t batch, int32_t bt_stride) {
    if (batch <= 0 || bt_stride <= KV_VERIFY_CHUNK_PAGES) return 0;
    return static_cast<size_t>(batch) * sizeof(uint64_t);     // one counter per request
}

int kv_verify_tags(const uint32_t* pool_tags, int32_t num_pages, const int32_t* block_table,
                   const uint32_t* expected_tags, int32_t bt_stride, const int32_t* seq_lens,
                   int32_t batch, int32_t page_size, uint8_t* abort_out, void* workspace,
                   size_t workspace_bytes, void* stream) {
    if (batch < 0 || num_pages < 0 || bt_stride < 0) return KV_ERR_SHAPE;
    if (page_size != KV_PAGE_SIZE) return KV_ERR_UNSUPPORTED;
    if (!grid_fits(batch, 1024)) return KV_ERR_SHAPE;     // one 1024-thread workgroup per request
    const int64_t chunks =
        bt_stride <= KV_VERIFY_CHUNK_PAGES
            ? 1
            : (static_cast<int64_t>(bt_stride) + KV_VERIFY_CHUNK_PAGES - 1) / KV_VERIFY_CHUNK_PAGES;
    const bool split = chunks > 1 && workspace != nullptr;
    if (split && !grid_fits(static_cast<int64_t>(batch) * chunks, 256)) return KV_ERR_SHAPE;
    if (batch == 0) return KV_OK;
    if (!block_table || !expected_tags || !seq_lens || !abort_out) return KV_ERR_NULL;
    if (!pool_tags && num_pages > 0) return KV_ERR_NULL;
    if (split && workspace_bytes < kv_verify_tags_workspace_bytes(batch, bt_stride))
        return KV_ERR_WORKSPACE;
    if (misaligned(pool_tags, 4) || misaligned(block_table, 4) || misaligned(expected_tags, 4) ||
        misaligned(seq_lens, 4) || (split && misaligned(workspace, 8)))
        return KV_ERR_ALIGN;
    return launch_status(kvfp8::launch_verify_tags(
        pool_tags, num_pages, block_table, expected_tags, bt_stride, seq_lens, batch, abort_out,
        split ? static_cast<uint64_t*>(workspace) : nullptr, static_cast<hipStream_t>(stream)));
}

int kv_append_quant(const void* k_new, const void* v_new, const int32_t* tok_seq,
                    const int32_t* tok_pos, int32_t n_tok, const int32_t* block_table,
                    int32_t bt_stride, int32_t batch, const float* k_scale, const float* v_scale,
                    uint8_t* k_pool, uint8_t* v_pool, int32_t num_pages, int32_t num_kv_heads,
                    int32_t head_dim, int32_t page_size, const uint8_t* abort, void* stream) {
    int st = check_append_common(k_new, v_new, tok_seq, tok_pos, n_tok, block_table, bt_stride,
                                 batch, k_pool, v_pool, num_pages, num_kv_heads, head_dim,
                                 page_size, abort);
    if (st != KV_OK || n_tok == 0) return st;
    if (!k_scale || !v_scale) return KV_ERR_NULL;
    if (misaligned(k_scale, 4) || misaligned(v_scale, 4)) return KV_ERR_ALIGN;
    return launch_status(kvfp8::launch_append(
        true, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), tok_seq,
        tok_pos, n_tok, block_table, bt_stride, batch, k_scale, v_scale, k_pool, v_pool,
        num_pages, num_kv_heads, abort, static_cast<hipStream_t>(stream)));
}

int kv_append_bf16(const void* k_new, const void* v_new, const int32_t* tok_seq,
                   const int32_t* tok_pos, int32_t n_tok, const int32_t* block_table,
                   int32_t bt_stride, int32_t batch, void* k_pool, void* v_pool,
                   int32_t num_pages, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                   const uint8_t* abort, void* stream) {
    int st = check_append_common(k_new, v_new, tok_seq, tok_pos, n_tok, block_table, bt_stride,
                                 batch, k_pool, v_pool, num_pages, num_kv_heads, head_dim,
                                 page_size, abort);
    if (st != KV_OK || n_tok == 0) return st;
    return launch_status(kvfp8::launch_append(
        false, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), tok_seq,
        tok_pos, n_tok, block_table, bt_stride, batch, nullptr, nullptr, k_pool, v_pool,
        num_pages, num_kv_heads, abort, static_cast<hipStream_t>(stream)));
}

int32_t paged_decode_attn_partition_tokens(int32_t batch, int32_t num_kv_heads,
                                           int32_t max_seq_len, int32_t partition_tokens,
                                           int32_t cache_dtype) {
    if (partition_tokens < 0) return KV_ERR_UNSUPPORTED;
    if (cache_dtype != KV_CACHE_FP8_E4M3 && cache_dtype != KV_CACHE_BF16)
        return KV_ERR_UNSUPPORTED;
    if (partition_tokens > 0) {
        if (partition_tokens % KV_PAGE_SIZE != 0 || partition_tokens > KV_MAX_PARTITION_TOKENS)
            return KV_ERR_UNSUPPORTED;
        return partition_tokens;
    }
    if (batch <= 0 || num_kv_heads <= 0 || max_seq_len <= 0) return 1024;
    return auto_partition(batch, num_kv_heads, max_seq_len, cache_dtype == KV_CACHE_FP8_E4M3);
}

size_t paged_decode_attn_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t max_seq_len, int32_t partition_tokens,
                                         int32_t cache_dtype) {
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0 ||
        head_dim != KV_HEAD_DIM)
        return 0;
    const int32_t pt = paged_decode_attn_partition_tokens(batch, num_kv_heads, max_seq_len,
                                                          partition_tokens, cache_dtype);
    if (pt <= 0) return 0;
    const int64_t parts = (static_cast<int64_t>(max_seq_len) + pt - 1) / pt;
    if (parts <= 1) return 0;
    // [slots][2] (max, sum), then [slots][head_dim] outputs
    return kvfp8::workspace_layout(batch, num_q_heads, parts).total;
}

int paged_decode_attn(const void* q, int32_t cache_dtype, const void* k_pool, const void* v_pool,
                      const float* k_scale, const float* v_scale, const int32_t* block_table,
                      int32_t bt_stride, const int32_t* seq_lens, int32_t max_seq_len,
                      const uint8_t* abort, float* out, float sm_scale, int32_t batch,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t page_size, int32_t num_pages, int32_t partition_tokens,
                      void* workspace, size_t workspace_bytes, void* stream) {
    // the pools are only read on this path
    return attn_impl(q, nullptr, nullptr, cache_dtype, const_cast<void*>(k_pool),
                     const_cast<void*>(v_pool), k_scale, v_scale, block_table, bt_stride,
                     seq_lens, max_seq_len, abort, out, sm_scale, batch, num_q_heads,
                     num_kv_heads, head_dim, page_size, num_pages, partition_tokens, workspace,
                     workspace_bytes, stream);
}

int paged_decode_attn_append(const void* q, const void* k_new, const void* v_new,
                             int32_t cache_dtype, void* k_pool, void* v_pool,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_table, int32_t bt_stride,
                             const int32_t* seq_lens, int32_t max_seq_len, const uint8_t* abort,
                             float* out, float sm_scale, int32_t batch, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                             int32_t num_pages, int32_t partition_tokens, void* workspace,
                             size_t workspace_bytes, void* stream) {
    if (batch > 0 && (!k_new || !v_new)) return KV_ERR_NULL;
    return attn_impl(q, k_new, v_new, cache_dtype, k_pool, v_pool, k_scale, v_scale,
                     block_table, bt_stride, seq_lens, max_seq_len, abort, out, sm_scale, batch,
                     num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                     partition_tokens, workspace, workspace_bytes, stream);
}

int paged_decode_attn_append_noalloc(const void* q, const void* k_new, const void* v_new,
                                     int32_t cache_dtype, void* k_pool, void* v_pool,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* block_table, int32_t bt_stride,
                                     const int32_t* seq_lens, int32_t max_seq_len,
                                     const uint8_t* abort, float* out, float sm_scale,
                                     int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t page_size, int32_t num_pages,
                                     int32_t partition_tokens, void* stream) {
    if (batch > 0 && (!k_new || !v_new)) return KV_ERR_NULL;
    return attn_impl(q, k_new, v_new, cache_dtype, k_pool, v_pool, k_scale, v_scale,
                     block_table, bt_stride, seq_lens, max_seq_len, abort, out, sm_scale, batch,
                     num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                     partition_tokens, nullptr, 0, stream, /*static_workspace=*/true);
}

int kv_amax_accumulate(const void* x, int64_t n_rows, int32_t num_kv_heads, int32_t head_dim,
                       float* amax_inout, void* stream) {
    if (n_rows < 0 || num_kv_heads <= 0) return KV_ERR_SHAPE;
    if (head_dim != KV_HEAD_DIM) return KV_ERR_UNSUPPORTED;
    if (n_rows == 0) return KV_OK;
    if (!x || !amax_inout) return KV_ERR_NULL;
    if (misaligned(x, 16) || misaligned(amax_inout, 4)) return KV_ERR_ALIGN;
    return launch_status(kvfp8::launch_amax(static_cast<const uint16_t*>(x), n_rows, num_kv_heads,
                                            amax_inout, static_cast<hipStream_t>(stream)));
}

int kv_scales_from_amax(const float* amax, int32_t n, float* scale_out, void* stream) {
    if (n < 0) return KV_ERR_SHAPE;
    if (n == 0) return KV_OK;
    if (!amax || !scale_out) return KV_ERR_NULL;
    if (misaligned(amax, 4) || misaligned(scale_out, 4)) return KV_ERR_ALIGN;
    return launch_status(kvfp8::launch_scales(amax, n, scale_out, static_cast<hipStream_t>(stream)));
}

int kv_ingest_prefill(const void* k_rows, const void* v_rows, int64_t n_rows,
                      const int32_t* row_start, const int32_t* seq_lens, int32_t batch,
                      int32_t max_seq_len, const int32_t* block_table, int32_t bt_stride,
                      int32_t cache_dtype, const float* k_scale, const float* v_scale,
                      void* k_pool, void* v_pool, int32_t num_pages, int32_t num_kv_heads,
                      int32_t head_dim, int32_t page_size, const uint8_t* abort, void* stream) {
    if (n_rows < 0 || batch < 0 || max_seq_len < 0 || bt_stride < 0 || num_pages < 0 ||
        num_kv_heads <= 0)
        return KV_ERR_SHAPE;
    if (head_dim != KV_HEAD_DIM || page_size != KV_PAGE_SIZE) return KV_ERR_UNSUPPORTED;
    if (cache_dtype != KV_CACHE_FP8_E4M3 && cache_dtype != KV_CACHE_BF16) return KV_ERR_UNSUPPORTED;
    if (batch == 0 || max_seq_len == 0) return KV_OK;
    const bool fp8 = cache_dtype == KV_CACHE_FP8_E4M3;
    if (!row_start || !seq_lens || !block_table || !k_pool || !v_pool) return KV_ERR_NULL;
    if (n_rows > 0 && (!k_rows || !v_rows)) return KV_ERR_NULL;
    if (fp8 && (!k_scale || !v_scale)) return KV_ERR_NULL;
    if (misaligned(k_rows, 16) || misaligned(v_rows, 16) || misaligned(k_pool, 16) ||
        misaligned(v_pool, 16) || misaligned(row_start, 4) || misaligned(seq_lens, 4) ||
        misaligned(block_table, 4) || (fp8 && (misaligned(k_scale, 4) || misaligned(v_scale, 4))))
        return KV_ERR_ALIGN;
    return launch_status(kvfp8::launch_ingest(
        fp8, static_cast<const uint16_t*>(k_rows), static_cast<const uint16_t*>(v_rows), n_rows,
        row_start, seq_lens, batch, max_seq_len, block_table, bt_stride, k_scale, v_scale, k_pool,
        v_pool, num_pages, num_kv_heads, abort, static_cast<hipStream_t>(stream)));
}

size_t wq_packed_bytes(int32_t n, int32_t k, int32_t format) {
    if (n < 0 || k < 0 || n % 16 || k % 128 || (format != WQ_INT4 && format != WQ_FP8_E4M3))
        return 0;
    return kvfp8::wq_packed_bytes(n, k, format == WQ_INT4);
}

int wq_quantize_pack(const void* w, int32_t n, int32_t k, int32_t format, void* packed,
                     float* scales, void* stream) {
    if (n < 0 || k < 0) return KV_ERR_SHAPE;
    if (n % 16 || k % 128) return KV_ERR_UNSUPPORTED;
    if (format != WQ_INT4 && format != WQ_FP8_E4M3) return KV_ERR_UNSUPPORTED;
    // one wavefront per (16-row tile, 128-input group), 4 per workgroup
    if (!grid_fits((static_cast<int64_t>(n / 16) * (k / 128) + 3) / 4, 256)) return KV_ERR_SHAPE;
    if (n == 0 || k == 0) return KV_OK;
    if (!w || !packed || !scales) return KV_ERR_NULL;
    if (misaligned(w, 16) || misaligned(packed, 16) || misaligned(scales, 16)) return KV_ERR_ALIGN;
    return launch_status(kvfp8::launch_wq_pack(format == WQ_INT4, static_cast<const uint16_t*>(w),
                                               n, k, static_cast<uint8_t*>(packed), scales,
                                               static_cast<hipStream_t>(stream)));
}

int wq_gemv(const void* x, int32_t m, const void* packed, const float* scales, int32_t n,
            int32_t k, int32_t format, float* y, void* stream) {
    if (m < 0 || n < 0 || k < 0) return KV_ERR_SHAPE;
    if (n % 16 || k % 128) return KV_ERR_UNSUPPORTED;
    if (format != WQ_INT4 && format != WQ_FP8_E4M3) return KV_ERR_UNSUPPORTED;
    // at most one workgroup per (64-row group, 128-input group)
    if (!grid_fits(static_cast<int64_t>((n / 16 + 3) / 4) * (k / 128), 256)) return KV_ERR_SHAPE;
    if (m == 0 || n == 0 || k == 0) return KV_OK;
    if (!x || !packed || !scales || !y) return KV_ERR_NULL;
    if (misaligned(x, 16) || misaligned(packed, 16) || misaligned(scales, 16) || misaligned(y, 16))
        return KV_ERR_ALIGN;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    for (int32_t m0 = 0; m0 < m; m0 += 64) {            // 64 activation rows per launch
        const int32_t rows = m - m0 < 64 ? m - m0 : 64;
        const int r = launch_status(kvfp8::launch_wq_gemv(
            format == WQ_INT4, static_cast<const uint16_t*>(x) + static_cast<size_t>(m0) * k, rows,
            static_cast<const uint8_t*>(packed), scales, n, k, y + static_cast<size_t>(m0) * n, st));
        if (r != KV_OK) return r;
    }
    return KV_OK;
}

}  // extern "C"
