// Argument validation of the C ABI (include/kvfp8.h), run on a host without
// a GPU under AddressSanitizer + UndefinedBehaviorSanitizer by
// tests/test_sanitizers.py. Every call below must be refused by validation
// with the stated status before anything is enqueued (a call that got through
// would return KV_ERR_LAUNCH here). Sizes include the int32 extremes, so the
// sizing arithmetic (partition counts, workspace bytes, grid limits) runs on
// values where a signed overflow would show. Prints "ok" and exits 0.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "kvfp8.h"

namespace {

int g_fail = 0;

void expect(const char* what, int got, int want) {
    if (got != want) {
        std::fprintf(stderr, "FAIL: %s returned %d, expected %d\n", what, got, want);
        ++g_fail;
    }
}

// A fake, aligned "device" address: never dereferenced, every call is refused first.
void* const A = reinterpret_cast<void*>(uintptr_t{1} << 20);
template <typename T>
T* P() { return static_cast<T*>(A); }

}  // namespace

int main() {
    const int32_t big[] = {INT32_MAX, INT32_MAX - 1, 1 << 30, 4194304, 16777216, -1, INT32_MIN};

    // tag check
    expect("verify page_size", kv_verify_tags(P<uint32_t>(), 10, P<int32_t>(), P<uint32_t>(), 4,
                                              P<int32_t>(), 2, 8, P<uint8_t>(), nullptr, 0,
                                              nullptr),
           KV_ERR_UNSUPPORTED);
    for (int32_t b : big)
        if (b > 4194303 || b < 0)
            expect("verify batch", kv_verify_tags(P<uint32_t>(), 10, P<int32_t>(), P<uint32_t>(), 4,
                                                  P<int32_t>(), b, 16, P<uint8_t>(), nullptr, 0,
                                                  nullptr),
                   KV_ERR_SHAPE);
    expect("verify null", kv_verify_tags(P<uint32_t>(), 10, nullptr, P<uint32_t>(), 4,
                                         P<int32_t>(), 2, 16, P<uint8_t>(), nullptr, 0, nullptr),
           KV_ERR_NULL);
    // the split check: its workgroup count at the extremes, and a short workspace
    for (int32_t b : {1, 2, 4096, 4194303})
        for (int32_t w : big)
            if (w > 0) {    // every such row is split, so the empty workspace is refused
                const int st = kv_verify_tags(P<uint32_t>(), 10, P<int32_t>(), P<uint32_t>(), w,
                                              P<int32_t>(), b, 16, P<uint8_t>(), A, 0, nullptr);
                if (st != KV_ERR_SHAPE && st != KV_ERR_WORKSPACE)
                    expect("verify split sizes", st, KV_ERR_SHAPE);
                (void)kv_verify_tags_workspace_bytes(b, w);
            }
    expect("verify workspace", kv_verify_tags(P<uint32_t>(), 10, P<int32_t>(), P<uint32_t>(), 5000,
                                              P<int32_t>(), 4, 16, P<uint8_t>(), A, 24, nullptr),
           KV_ERR_WORKSPACE);

    // append
    for (int32_t n : big)
        if (n > 16777215 || n < 0)
            expect("append n_tok", kv_append_quant(A, A, P<int32_t>(), P<int32_t>(), n, P<int32_t>(),
                                                   4, 2, P<float>(), P<float>(), P<uint8_t>(),
                                                   P<uint8_t>(), 10, 8, 128, 16, nullptr, nullptr),
                   KV_ERR_SHAPE);
    expect("append head_dim", kv_append_bf16(A, A, P<int32_t>(), P<int32_t>(), 3, P<int32_t>(), 4, 2,
                                             A, A, 10, 8, 64, 16, nullptr, nullptr),
           KV_ERR_UNSUPPORTED);
    expect("append align", kv_append_quant(A, A, P<int32_t>(), P<int32_t>(), 3, P<int32_t>(), 4, 2,
                                           P<float>(), P<float>(), P<uint8_t>() + 4, P<uint8_t>(),
                                           10, 8, 128, 16, nullptr, nullptr),
           KV_ERR_ALIGN);

    // attention: sizing at the extremes, then refusals
    for (int32_t cd : {KV_CACHE_FP8_E4M3, KV_CACHE_BF16})
        for (int32_t b : big)
            for (int32_t L : big) {
                const int32_t pt = paged_decode_attn_partition_tokens(b, 8, L, 0, cd);
                if (pt != KV_ERR_UNSUPPORTED &&
                    (pt < 16 || pt > KV_MAX_PARTITION_TOKENS || pt % 16))
                    expect("partition tokens range", pt, 512);
                (void)paged_decode_attn_workspace_bytes(b, 64, 8, 128, L, 0, cd);
                (void)paged_decode_attn_workspace_bytes(b, INT32_MAX, 1, 128, L, 16, cd);
                (void)paged_decode_attn_workspace_bytes(b, 64, INT32_MAX, 128, L, 16384, cd);
            }
    expect("partition tokens dtype", paged_decode_attn_partition_tokens(4, 8, 1000, 0, 7),
           KV_ERR_UNSUPPORTED);
    if (paged_decode_attn_workspace_bytes(4, 64, 8, 128, 100000, 0, 7) != 0)
        expect("workspace dtype", 1, 0);
    expect("attn partitions", paged_decode_attn(A, 0, A, A, P<float>(), P<float>(), P<int32_t>(), 8,
                                                 P<int32_t>(), INT32_MAX, nullptr, P<float>(), 0.1f,
                                                 4, 64, 8, 128, 16, 10, 16, A, 1 << 20, nullptr),
           KV_ERR_UNSUPPORTED);
    expect("attn grid", paged_decode_attn(A, 0, A, A, P<float>(), P<float>(), P<int32_t>(), 8,
                                          P<int32_t>(), 1, nullptr, P<float>(), 0.1f, INT32_MAX, 64,
                                          8, 128, 16, 10, 0, nullptr, 0, nullptr),
           KV_ERR_SHAPE);
    expect("attn group", paged_decode_attn(A, 0, A, A, P<float>(), P<float>(), P<int32_t>(), 8,
                                           P<int32_t>(), 100, nullptr, P<float>(), 0.1f, 4, 64, 2,
                                           128, 16, 10, 0, nullptr, 0, nullptr),
           KV_ERR_UNSUPPORTED);
    expect("attn sm_scale", paged_decode_attn(A, 0, A, A, P<float>(), P<float>(), P<int32_t>(), 8,
                                              P<int32_t>(), 100, nullptr, P<float>(), -1.0f, 4, 64,
                                              8, 128, 16, 10, 0, nullptr, 0, nullptr),
           KV_ERR_UNSUPPORTED);
    expect("attn workspace", paged_decode_attn(A, 0, A, A, P<float>(), P<float>(), P<int32_t>(), 8,
                                               P<int32_t>(), 100000, nullptr, P<float>(), 0.1f, 4,
                                               64, 8, 128, 16, 10, 512, A, 64, nullptr),
           KV_ERR_WORKSPACE);
    expect("fused null", paged_decode_attn_append(A, nullptr, A, 0, A, A, P<float>(), P<float>(),
                                                  P<int32_t>(), 8, P<int32_t>(), 100, nullptr,
                                                  P<float>(), 0.1f, 4, 64, 8, 128, 16, 10, 0,
                                                  nullptr, 0, nullptr),
           KV_ERR_NULL);

    // the no-alloc entry point: refused before its scratch is looked up
    expect("noalloc scratch", paged_decode_attn_append_noalloc(
               A, A, A, 0, A, A, P<float>(), P<float>(), P<int32_t>(), 8193, P<int32_t>(), 131073,
               nullptr, P<float>(), 0.1f, 16, 64, 8, 128, 16, 10, 512, nullptr),
           KV_ERR_WORKSPACE);
    expect("noalloc null", paged_decode_attn_append_noalloc(
               A, nullptr, A, 0, A, A, P<float>(), P<float>(), P<int32_t>(), 8, P<int32_t>(), 100,
               nullptr, P<float>(), 0.1f, 4, 64, 8, 128, 16, 10, 0, nullptr),
           KV_ERR_NULL);
    expect("noalloc group", paged_decode_attn_append_noalloc(
               A, A, A, 0, A, A, P<float>(), P<float>(), P<int32_t>(), 8, P<int32_t>(), 100,
               nullptr, P<float>(), 0.1f, 4, 64, 2, 128, 16, 10, 0, nullptr),
           KV_ERR_UNSUPPORTED);

    // prefill ingest, weight GEMV
    expect("ingest dtype", kv_ingest_prefill(A, A, 10, P<int32_t>(), P<int32_t>(), 2, 10, P<int32_t>(),
                                             4, 5, P<float>(), P<float>(), A, A, 10, 8, 128, 16,
                                             nullptr, nullptr),
           KV_ERR_UNSUPPORTED);
    expect("amax rows", kv_amax_accumulate(A, -1, 8, 128, P<float>(), nullptr), KV_ERR_SHAPE);
    expect("scales null", kv_scales_from_amax(nullptr, 8, P<float>(), nullptr), KV_ERR_NULL);
    expect("pack rows", wq_quantize_pack(A, 1000, 128, WQ_INT4, A, P<float>(), nullptr),
           KV_ERR_UNSUPPORTED);
    expect("pack huge", wq_quantize_pack(A, INT32_MAX - 15, 1 << 20, WQ_INT4, A, P<float>(), nullptr),
           KV_ERR_SHAPE);
    expect("pack grid", wq_quantize_pack(A, 1 << 30, 1 << 30, WQ_INT4, A, P<float>(), nullptr),
           KV_ERR_SHAPE);
    expect("gemv grid", wq_gemv(A, 4, A, P<float>(), 1 << 30, 1 << 30, WQ_INT4, P<float>(), nullptr),
           KV_ERR_SHAPE);
    if (wq_packed_bytes(INT32_MAX, INT32_MAX, WQ_FP8_E4M3) != 0 &&
        wq_packed_bytes(1 << 30, 1 << 30, WQ_FP8_E4M3) == 0)
        expect("packed bytes", 0, 1);
    for (int s = -9; s <= 1; ++s)
        if (kv_status_str(s) == nullptr) expect("status string", 0, 1);

    if (g_fail) return 1;
    std::printf("ok\n");
    return 0;
}
