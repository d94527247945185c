// Internal host-side launchers. Arguments are already validated by the C-ABI
// layer (kvfp8_api.hip); each launcher only enqueues its kernels on `stream`
// and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvfp8 {

// Pages of a request's row that one workgroup of the split tag check covers.
constexpr int kVerifyChunkPages = 2048;

// counters: nullptr (one workgroup per whole row), or batch zero-filled 64-bit
// words (rows split into chunks of kVerifyChunkPages pages, one workgroup each).
hipError_t launch_verify_tags(const uint32_t* pool_tags, int32_t num_pages,
                              const int32_t* block_table, const uint32_t* expected_tags,
                              int32_t bt_stride, const int32_t* seq_lens, int32_t batch,
                              uint8_t* abort_out, uint64_t* counters, hipStream_t stream);

hipError_t launch_append(bool fp8, const uint16_t* k_new, const uint16_t* v_new,
                         const int32_t* tok_seq, const int32_t* tok_pos, int32_t n_tok,
                         const int32_t* block_table, int32_t bt_stride, int32_t batch,
                         const float* k_scale, const float* v_scale, void* k_pool,
                         void* v_pool, int32_t num_pages, int32_t num_kv_heads,
                         const uint8_t* abort, hipStream_t stream);

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* k_new;      // non-null: append the token L-1 first (fused path)
    const uint16_t* v_new;
    void* k_pool;
    void* v_pool;
    const float* k_scale;
    const float* v_scale;
    const int32_t* block_table;
    int32_t bt_stride;
    const int32_t* seq_lens;
    int32_t max_seq_len;
    const uint8_t* abort;
    float* out;
    float sm_scale;
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t num_pages;
    int32_t partition_tokens;   // resolved, > 0
    int32_t num_partitions;     // ceil(max_seq_len / partition_tokens), >= 1
    float* part_ml;             // [batch][Hq][partial_slots(num_partitions)][2], or null if 1 partition
    float* part_acc;            // [batch][Hq][partial_slots(num_partitions)][128]
};

// Split-K partial slots per (request, query head): one per partition, plus
// one more that the wave-mode kernel uses when a wavefront's share starts
// inside a request's last partition (the slot after that partition).
__host__ __device__ constexpr int64_t partial_slots(int64_t num_partitions) {
    return num_partitions + 1;
}

// Workspace layout of the attention calls with more than one partition:
// the (max, sum) pairs, then the partial outputs from the next 256-byte
// boundary.
struct WorkspaceLayout {
    size_t ml;                  // byte offsets
    size_t acc;
    size_t total;
};

inline WorkspaceLayout workspace_layout(int64_t batch, int64_t num_q_heads,
                                        int64_t num_partitions) {
    const auto up = [](size_t n) { return (n + 255) / 256 * 256; };
    const size_t slots = static_cast<size_t>(batch) * num_q_heads * partial_slots(num_partitions);
    WorkspaceLayout w{};
    w.ml = 0;
    w.acc = up(slots * 2 * sizeof(float));
    w.total = w.acc + slots * 128 * sizeof(float);
    return w;
}

hipError_t launch_decode_attn(bool fp8, const AttnArgs& a, hipStream_t stream);

hipError_t launch_amax(const uint16_t* x, int64_t n_rows, int32_t hkv, float* amax_inout,
                       hipStream_t stream);

hipError_t launch_scales(const float* amax, int32_t n, float* out, hipStream_t stream);

hipError_t launch_ingest(bool fp8, const uint16_t* k_rows, const uint16_t* v_rows,
                         int64_t n_rows, const int32_t* row_start, const int32_t* seq_lens,
                         int32_t batch, int32_t max_seq_len, const int32_t* block_table,
                         int32_t bt_stride, const float* k_scale, const float* v_scale,
                         void* k_pool, void* v_pool, int32_t num_pages, int32_t num_kv_heads,
                         const uint8_t* abort, hipStream_t stream);

size_t wq_packed_bytes(int32_t n, int32_t k, bool int4);

hipError_t launch_wq_pack(bool int4, const uint16_t* w, int32_t n, int32_t k, uint8_t* packed,
                          float* scales, hipStream_t stream);

hipError_t launch_wq_gemv(bool int4, const uint16_t* x, int32_t m_rows, const uint8_t* packed,
                          const float* scales, int32_t n, int32_t k, float* y,
                          hipStream_t stream);

}  // namespace kvfp8
