// Page-tag verification and append (quantize-on-append / bf16 copy) kernels.
//
// Tag check: the pages describe a separate batched check that compares each
// request's recorded (page, tag) pairs with the pool's current tags before
// supported decode operations read, aborting just the mismatching request
// (remio.ai/it "Il serving di modelli più piccoli di Cloudflare ...", sections
// "Cosa ha cambiato Cloudflare per Kimi e GLM" and "La sicurezza della cache
// KV condivisa diventa una questione di produzione").
//
// Append: the cache is stored as FP8 e4m3 instead of BF16 (same page, section
// "Cosa ha cambiato ..."); each new token's K/V row is divided by its
// (layer, KV head) scale and rounded to e4m3 on the way into its page slot.
#include "kv_device.h"
#include "kv_launch.h"

namespace kvfp8 {

// ---------------------------------------------------------------------------
// kv_verify_tags: one 1024-thread workgroup per request. Each thread checks up
// to 8 logical pages per sweep and one sweep covers 8192 pages (131,072
// tokens). A sweep is branch-free: the table entries and expected tags are
// loaded with indices clamped into the request's row, then every pool tag is
// gathered (an out-of-range id reads tag 0 instead, and is flagged anyway),
// so all loads of a step are in flight together. The first sweep's table
// loads are clamped into the table row (bt_stride entries) rather than the
// request's pages, so they go out together with the length load and the
// check costs two memory round trips, not three. The workgroup ORs the
// per-thread verdicts and one thread writes the request's flag.
// ---------------------------------------------------------------------------
constexpr int kVerifyThreads = 1024;
constexpr int kVerifyUnroll = 8;

__global__ __launch_bounds__(kVerifyThreads) void verify_tags_kernel(
    const uint32_t* __restrict__ pool_tags, int32_t num_pages,
    const int32_t* __restrict__ block_table, const uint32_t* __restrict__ expected_tags,
    int32_t bt_stride, const int32_t* __restrict__ seq_lens, uint8_t* __restrict__ abort_out) {
    const int b = blockIdx.x;
    const int32_t* bt_row = block_table + static_cast<size_t>(b) * bt_stride;
    const uint32_t* ex_row = expected_tags + static_cast<size_t>(b) * bt_stride;
    int32_t page[kVerifyUnroll];
    uint32_t want[kVerifyUnroll];
    if (bt_stride > 0) {
#pragma unroll
        for (int u = 0; u < kVerifyUnroll; ++u) {
            const int j = min(u * kVerifyThreads + static_cast<int>(threadIdx.x), bt_stride - 1);
            page[u] = bt_row[j];
            want[u] = ex_row[j];
        }
    }
    const int L = seq_lens[b];
    int bad = 0;
    int64_t npages = 0;
    if (L < 0) {
        bad = 1;
    } else {
        npages = (static_cast<int64_t>(L) + kPage - 1) / kPage;
        if (npages > bt_stride) bad = 1;
        if (npages > 0 && num_pages <= 0) bad = 1;       // no page can be valid (no tags to read)
    }
    if (!bad && npages > 0) {
        for (int64_t base = 0; base < npages; base += kVerifyThreads * kVerifyUnroll) {
            if (base > 0) {
#pragma unroll
                for (int u = 0; u < kVerifyUnroll; ++u) {
                    const int64_t j = min(base + u * kVerifyThreads + threadIdx.x, npages - 1);
                    page[u] = bt_row[j];
                    want[u] = ex_row[j];
                }
            }
            uint32_t have[kVerifyUnroll];
#pragma unroll
            for (int u = 0; u < kVerifyUnroll; ++u) {
                const int64_t j = base + u * kVerifyThreads + threadIdx.x;
                const int32_t p = page[u];
                have[u] = pool_tags[(j < npages && p >= 0 && p < num_pages) ? p : 0];
            }
#pragma unroll
            for (int u = 0; u < kVerifyUnroll; ++u) {
                const int64_t j = base + u * kVerifyThreads + threadIdx.x;
                const int32_t p = page[u];
                const bool wrong = p < 0 || p >= num_pages || have[u] != want[u];
                bad |= (j < npages && wrong) ? 1 : 0;
            }
        }
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) abort_out[b] = bad ? 1 : 0;
}

// ---------------------------------------------------------------------------
// Split tag check: workgroup (b, c) of 256 threads checks pages
// [c * 2048, (c + 1) * 2048) of request b's row, 8 per thread, all loads of a
// thread in flight together as above. A row of n chunks (n = 1 for a refused
// request; workgroups past a row's n exit at once) with n == 1 writes its
// flag directly. Otherwise each of the n workgroups adds 1 to the request's
// 64-bit counter, plus 2^32 if it found a mismatch, with one relaxed device-
// scope atomic; the workgroup that brings the count to n writes the flag from
// the sum it read and stores 0 back, so the counters start every call at zero
// and the flag is still overwritten, never accumulated. The verdict travels
// inside the atomic, so no other memory has to become visible.
// ---------------------------------------------------------------------------
constexpr int kVerifySplitThreads = 256;
constexpr int kVerifySplitUnroll = kVerifyChunkPages / kVerifySplitThreads;
static_assert(kVerifySplitUnroll * kVerifySplitThreads == kVerifyChunkPages, "chunk shape");

__global__ __launch_bounds__(kVerifySplitThreads) void verify_tags_split_kernel(
    const uint32_t* __restrict__ pool_tags, int32_t num_pages,
    const int32_t* __restrict__ block_table, const uint32_t* __restrict__ expected_tags,
    int32_t bt_stride, const int32_t* __restrict__ seq_lens, uint8_t* __restrict__ abort_out,
    uint64_t* __restrict__ counters, int32_t chunks_per_row) {
    const int b = static_cast<int>(blockIdx.x / static_cast<uint32_t>(chunks_per_row));
    const int c = static_cast<int>(blockIdx.x % static_cast<uint32_t>(chunks_per_row));
    const int64_t j0 = static_cast<int64_t>(c) * kVerifyChunkPages + threadIdx.x;
    const int32_t* bt_row = block_table + static_cast<size_t>(b) * bt_stride;
    const uint32_t* ex_row = expected_tags + static_cast<size_t>(b) * bt_stride;
    // this chunk's table entries, clamped into the row, go out with the length
    int32_t page[kVerifySplitUnroll];
    uint32_t want[kVerifySplitUnroll];
    if (bt_stride > 0) {
#pragma unroll
        for (int u = 0; u < kVerifySplitUnroll; ++u) {
            const int64_t j = min(j0 + u * kVerifySplitThreads, static_cast<int64_t>(bt_stride) - 1);
            page[u] = bt_row[j];
            want[u] = ex_row[j];
        }
    }
    const int L = seq_lens[b];
    int bad = 0;
    int64_t npages = 0;
    if (L < 0) {
        bad = 1;
    } else {
        npages = (static_cast<int64_t>(L) + kPage - 1) / kPage;
        if (npages > bt_stride) bad = 1;
        if (npages > 0 && num_pages <= 0) bad = 1;
    }
    const int64_t n_chunks =
        bad ? 1 : max(int64_t{1}, (npages + kVerifyChunkPages - 1) / kVerifyChunkPages);
    if (c >= n_chunks) return;                                // uniform per workgroup
    if (!bad) {
        uint32_t have[kVerifySplitUnroll];
#pragma unroll
        for (int u = 0; u < kVerifySplitUnroll; ++u) {
            const int64_t j = j0 + u * kVerifySplitThreads;
            const int32_t p = page[u];
            have[u] = pool_tags[(j < npages && p >= 0 && p < num_pages) ? p : 0];
        }
#pragma unroll
        for (int u = 0; u < kVerifySplitUnroll; ++u) {
            const int64_t j = j0 + u * kVerifySplitThreads;
            const int32_t p = page[u];
            const bool wrong = p < 0 || p >= num_pages || have[u] != want[u];
            bad |= (j < npages && wrong) ? 1 : 0;
        }
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x != 0) return;
    if (n_chunks == 1) {
        abort_out[b] = bad ? 1 : 0;
        return;
    }
    const uint64_t add = 1u + (bad ? (uint64_t{1} << 32) : 0u);
    const uint64_t old = __hip_atomic_fetch_add(counters + b, add, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    if (static_cast<int64_t>(old & 0xFFFFFFFFu) + 1 == n_chunks) {
        abort_out[b] = ((old >> 32) != 0 || bad) ? 1 : 0;
        __hip_atomic_store(counters + b, uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

hipError_t launch_verify_tags(const uint32_t* pool_tags, int32_t num_pages,
                              const int32_t* block_table, const uint32_t* expected_tags,
                              int32_t bt_stride, const int32_t* seq_lens, int32_t batch,
                              uint8_t* abort_out, uint64_t* counters, hipStream_t stream) {
    const int64_t chunks = bt_stride <= kVerifyChunkPages
                               ? 1
                               : (static_cast<int64_t>(bt_stride) + kVerifyChunkPages - 1) /
                                     kVerifyChunkPages;
    if (chunks == 1 || counters != nullptr) {
        hipLaunchKernelGGL(verify_tags_split_kernel,
                           dim3(static_cast<uint32_t>(batch * chunks)), dim3(kVerifySplitThreads),
                           0, stream, pool_tags, num_pages, block_table, expected_tags, bt_stride,
                           seq_lens, abort_out, counters, static_cast<int32_t>(chunks));
    } else {
        hipLaunchKernelGGL(verify_tags_kernel, dim3(batch), dim3(kVerifyThreads), 0, stream,
                           pool_tags, num_pages, block_table, expected_tags, bt_stride, seq_lens,
                           abort_out);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Append. Grid: x = token n, y = slice of the token's (K|V, head, 4-dim group)
// work items; each thread handles 4 consecutive dims of one head of K or V.
// FP8: x / s rounded to fp32 with round-to-odd (correctly rounded division
// plus the sign of the exact fma remainder), clamp to +-448, then the
// hardware round-to-nearest-even convert; together this is round-to-nearest-
// even of the exact quotient. BF16: stored as is.
// ---------------------------------------------------------------------------
constexpr int kAppendThreads = 256;

template <bool FP8>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ tok_seq, const int32_t* __restrict__ tok_pos,
    const int32_t* __restrict__ block_table, int32_t bt_stride, int32_t batch,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool, int32_t num_pages,
    int32_t num_kv_heads, const uint8_t* __restrict__ abort) {
    const int n = blockIdx.x;
    const int items_per_kind = num_kv_heads * (kDim / 4);
    const int item = blockIdx.y * kAppendThreads + threadIdx.x;
    if (item >= 2 * items_per_kind) return;
    const int b = tok_seq[n];
    const int t = tok_pos[n];
    if (b < 0 || b >= batch || t < 0) return;
    if (abort != nullptr && abort[b] != 0) return;
    const int j = t / kPage;
    if (j >= bt_stride) return;
    const int page = block_table[static_cast<size_t>(b) * bt_stride + j];
    if (page < 0 || page >= num_pages) return;

    const bool is_v = item >= items_per_kind;
    const int rem = is_v ? item - items_per_kind : item;
    const int g = rem / (kDim / 4);
    const int d = (rem % (kDim / 4)) * 4;
    const int slot = t % kPage;
    const uint16_t* src = (is_v ? v_new : k_new) +
                          (static_cast<size_t>(n) * num_kv_heads + g) * kDim + d;
    const u32x2 raw = *reinterpret_cast<const u32x2*>(src);
    const size_t tile = static_cast<size_t>(page) * num_kv_heads + g;

    const float s = FP8 ? (is_v ? v_scale : k_scale)[g] : 1.0f;
    uint8_t* base = (is_v ? v_pool : k_pool) + tile * (FP8 ? kTileFp8 : kTileBf16);
    store_token_quad<FP8>(is_v, raw, s, base, slot, d);
}

hipError_t launch_append(bool fp8, const uint16_t* k_new, const uint16_t* v_new,
                         const int32_t* tok_seq, const int32_t* tok_pos, int32_t n_tok,
                         const int32_t* block_table, int32_t bt_stride, int32_t batch,
                         const float* k_scale, const float* v_scale, void* k_pool,
                         void* v_pool, int32_t num_pages, int32_t num_kv_heads,
                         const uint8_t* abort, hipStream_t stream) {
    const int items = 2 * num_kv_heads * (kDim / 4);
    const dim3 grid(n_tok, (items + kAppendThreads - 1) / kAppendThreads);
    if (fp8) {
        hipLaunchKernelGGL(append_kernel<true>, grid, dim3(kAppendThreads), 0, stream, k_new,
                           v_new, tok_seq, tok_pos, block_table, bt_stride, batch, k_scale,
                           v_scale, static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool),
                           num_pages, num_kv_heads, abort);
    } else {
        hipLaunchKernelGGL(append_kernel<false>, grid, dim3(kAppendThreads), 0, stream, k_new,
                           v_new, tok_seq, tok_pos, block_table, bt_stride, batch, k_scale,
                           v_scale, static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool),
                           num_pages, num_kv_heads, abort);
    }
    return hipGetLastError();
}

}  // namespace kvfp8
