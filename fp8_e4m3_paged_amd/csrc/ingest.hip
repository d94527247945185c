// Prefill ingest: the handoff of a prompt's BF16 keys and values into the
// decode cache. The pages (remio.ai/it "Il serving di modelli più piccoli di
// Cloudflare riduce la memoria, ma la sicurezza diventa la prova decisiva",
// section "Cosa ha cambiato Cloudflare per Kimi e GLM") run prefill and
// decode in separate pools: prefill builds a prompt's initial cache state in
// BF16, decode reads the smaller FP8 cache. Three kernels serve that handoff:
//
//  * amax_kernel: per-KV-head max |x| over the finite bf16 values of a
//    packed [rows][Hkv][128] tensor, accumulated into an fp32 array with one
//    atomic max per 16-lane group (non-negative floats order like their bits);
//  * scales_kernel: scale = fp32(amax / 448) (correctly rounded division),
//    raised to the smallest normal fp32, 1.0 for amax = 0 or non-finite;
//  * ingest_kernel<FP8>: whole (page, head) tiles of every prompt. Each lane
//    builds exactly the 16-byte chunks that the tile layout places at
//    16 * lane (+ 1 KiB per chunk), so every store is a full, coalesced
//    16-byte write of the 2 KiB (FP8) or 4 KiB (BF16) tile; slots past the
//    prompt's end are written as zeros. FP8 codes are those of the exact
//    quotient x / s; a wavefront whose head scale and values allow it
//    (almost always) forms them from the reciprocal and a Newton step
//    instead of an IEEE division, which made the writer ALU-bound.
#include <algorithm>
#include <type_traits>

#include "kv_device.h"
#include "kv_launch.h"

namespace kvfp8 {

// ---------------------------------------------------------------------------
// amax
// ---------------------------------------------------------------------------
constexpr int kAmaxThreads = 256;

__device__ __forceinline__ uint32_t finite_mag_max(uint32_t m, uint32_t w) {
    const uint32_t lo = w & 0x7FFFu;
    const uint32_t hi = (w >> 16) & 0x7FFFu;
    m = lo < 0x7F80u ? max(m, lo) : m;     // exponent all ones: +-Inf or NaN, skipped
    return hi < 0x7F80u ? max(m, hi) : m;
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Grid-stride over the 16-byte vectors of x, one load in flight per lane per
// step (measured faster than several 8 MiB apart); the stride is a multiple
// of 16 * hkv, so vector v always belongs to head (v / 16) % hkv and each
// thread keeps one running maximum. The maximum is taken first over all
// magnitudes as packed 16-bit lanes (two instructions per word); only a
// thread whose maximum is an Inf or NaN pattern scans its vectors again
// skipping those. The 16 groups of 16 lanes of a workgroup are combined per
// head in LDS, then one atomic max per head and workgroup (non-negative
// floats order like their bits).
__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(const u32x4* __restrict__ x,
                                                            int64_t n_vec, int32_t hkv,
                                                            uint32_t* __restrict__ amax_bits) {
    const int64_t first = static_cast<int64_t>(blockIdx.x) * kAmaxThreads + threadIdx.x;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kAmaxThreads;
    u16x2 mm = {0, 0};
    for (int64_t v = first; v < n_vec; v += stride) {
        const u32x4 w = __builtin_nontemporal_load(x + v);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            mm = __builtin_elementwise_max(mm, __builtin_bit_cast(u16x2, w[e] & 0x7FFF7FFFu));
    }
    uint32_t m = max(static_cast<uint32_t>(mm[0]), static_cast<uint32_t>(mm[1]));
    if (m >= 0x7F80u) {                    // rare: this thread saw +-Inf or NaN
        m = 0;
        for (int64_t v = first; v < n_vec; v += stride) {
            const u32x4 w = x[v];
#pragma unroll
            for (int e = 0; e < 4; ++e) m = finite_mag_max(m, w[e]);
        }
    }
    // the 16 lanes of a group cover one 256-byte head row segment: same head
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), o)));
    constexpr int kGroups = kAmaxThreads / 16;
    __shared__ uint32_t sm[kGroups];
    if ((threadIdx.x & 15) == 0) sm[threadIdx.x / 16] = m;
    __syncthreads();
    if (threadIdx.x < kGroups) {
        // group q's head is (16 blockIdx + q) % hkv; the first group of each head combines
        const int q = threadIdx.x;
        const int base = static_cast<int>((static_cast<int64_t>(blockIdx.x) * kGroups) % hkv);
        const int gq = (base + q) % hkv;
        if (q < hkv) {
            uint32_t r = 0;
            for (int j = q; j < kGroups; j += hkv) r = max(r, sm[j]);
            if (r != 0) atomicMax(amax_bits + gq, r << 16);
        }
    }
}

__global__ void scales_kernel(const float* __restrict__ amax, int32_t n, float* __restrict__ out) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
        const float a = amax[i];
        float s = 1.0f;
        if (a > 0.0f && a < INFINITY) s = fmaxf(a / 448.0f, 1.17549435082228750797e-38f);
        out[i] = s;
    }
}

// ---------------------------------------------------------------------------
// ingest
// ---------------------------------------------------------------------------
// The same codes as encode4_e4m3(div_round_odd(x_i, s)), without a division,
// for scales s in [2^-63, 2^63] with inv = 1 / s, and |x_i| <= 2^63 (so NaN
// and infinities are excluded and no quotient overflows):
//  * y0 = |x| inv is within ~2 ulp of the exact quotient; one Newton step
//    y1 = y0 + (|x| - y0 s) inv is then within one ulp of it (a faithful
//    rounding), and the remainder |x| - y1 s of a faithful quotient is
//    exactly representable, so its fma is exact;
//  * as in div_round_odd, a negative remainder steps the magnitude down one
//    ulp and any nonzero one sets the last bit (round-to-odd); the 448 clamp
//    and the sign of x are applied to the bits, then the hardware converts.
// In that range every quotient that can round to a nonzero code stays a
// normal float with a normal remainder; smaller ones round to zero however
// they are approximated.
__device__ __forceinline__ bool recip_quotient_ok(float s) {
    return s >= 0x1p-63f && s <= 0x1p63f;
}
constexpr uint16_t kRecipMaxMagBits = 0x5F00;      // bf16 magnitude bits of 2^63

__device__ __forceinline__ float quot_round_odd_clamped(float x, float s, float inv) {
    const float ax = fabsf(x);
    const float y0 = ax * inv;
    const float y1 = fmaf(fmaf(-y0, s, ax), inv, y0);
    const uint32_t rb = __float_as_uint(fmaf(-y1, s, ax));         // exact remainder
    uint32_t u = __float_as_uint(y1) + static_cast<uint32_t>(static_cast<int32_t>(rb) >> 31);
    u |= min(rb, 1u);
    u = min(u, 0x43E00000u);                                        // 448.0f
    return __uint_as_float(u | (__float_as_uint(x) & 0x80000000u));
}

__device__ __forceinline__ uint32_t encode4_e4m3_recip(float x0, float x1, float x2, float x3,
                                                       float s, float inv) {
    const uint32_t pk = __builtin_amdgcn_cvt_pk_fp8_f32(quot_round_odd_clamped(x0, s, inv),
                                                        quot_round_odd_clamped(x1, s, inv), 0u, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(quot_round_odd_clamped(x2, s, inv),
                                           quot_round_odd_clamped(x3, s, inv), pk, true);
}

// Running maximum of the magnitude bits of packed bf16 pairs (two 16-bit
// lanes), to check |x| <= 2^63 for a whole block before taking the
// reciprocal path.
__device__ __forceinline__ u16x2 bf16x2_max_mag(u16x2 m, uint32_t w) {
    return __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu));
}
__device__ __forceinline__ bool bf16x2_recip_range(u16x2 m) {
    return m[0] <= kRecipMaxMagBits && m[1] <= kRecipMaxMagBits;
}

// Four floats x_i -> the e4m3 codes of x_i / s: through the reciprocal when
// RECIP (the caller checked recip_quotient_ok(s) and |x_i| <= 2^63), else
// by division.
template <bool RECIP>
__device__ __forceinline__ uint32_t quant4_e4m3(float x0, float x1, float x2, float x3, float s,
                                                float inv) {
    if constexpr (RECIP) {
        return encode4_e4m3_recip(x0, x1, x2, x3, s, inv);
    } else {
        return encode4_e4m3(div_round_odd(x0, s), div_round_odd(x1, s), div_round_odd(x2, s),
                            div_round_odd(x3, s));
    }
}

constexpr int kIngestWaves = 4;
// One head's K rows, then its V rows, staged in LDS per wavefront (16 tokens
// x 128 bf16), rows padded to 272 bytes so V's transposed reads (4 token
// groups x 16 dims) hit disjoint banks and the 16-byte accesses stay aligned.
// Global loads read whole rows, each byte once, and the next head's rows are
// loaded into registers while the current head is encoded.
constexpr int kVRowHalves = 136;

// Orders one wavefront's LDS writes before its reads (and reads before the
// next writes): LDS operations of a wave complete in order, so only the
// compiler has to be kept from moving them.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Whether every lane of the wavefront holds only |x| <= 2^63 among one
// head's rows (no NaN or infinity): then the reciprocal encoder is exact.
__device__ __forceinline__ bool wave_recip_range(const u32x4 (&w)[4]) {
    u16x2 m = {0, 0};
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = bf16x2_max_mag(m, w[k][e]);
    return __builtin_amdgcn_ballot_w64(!bf16x2_recip_range(m)) == 0;
}

// 16 bytes of a pool tile. The pages are written once and not read again by
// this launch, so the store is non-temporal (streamed past the caches).
__device__ __forceinline__ void store_stream(uint8_t* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Page j of request b (one workgroup; each wavefront takes KV heads wave,
// wave + 4, ... and uses only its own LDS block).
template <bool FP8>
__device__ __forceinline__ void ingest_page(
    int b, int j, const uint16_t* __restrict__ k_rows, const uint16_t* __restrict__ v_rows,
    int64_t n_rows, const int32_t* __restrict__ row_start, const int32_t* __restrict__ seq_lens,
    int32_t max_seq_len, const int32_t* __restrict__ block_table, int32_t bt_stride,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool, int32_t num_pages, int32_t hkv,
    const uint8_t* __restrict__ abort, uint16_t (*sx)[kVRowHalves]) {
    const int L = seq_lens[b];
    if (abort != nullptr && abort[b] != 0) return;
    if (L <= 0 || L > max_seq_len || (static_cast<int64_t>(L) + kPage - 1) / kPage > bt_stride)
        return;
    if (j * kPage >= L) return;
    const int64_t r0 = row_start[b];
    if (r0 < 0 || r0 + L > n_rows) return;                   // rows outside the inputs
    const int page = block_table[static_cast<size_t>(b) * bt_stride + j];
    if (page < 0 || page >= num_pages) return;
    const int n = min(kPage, L - j * kPage);                  // live slots of this page
    const size_t row0 = static_cast<size_t>(r0) + static_cast<size_t>(j) * kPage;
    const size_t row_elems = static_cast<size_t>(hkv) * kDim;

    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    const int m = lane % 16;          // K: token of the lane; V: dim within a 16-dim chunk
    const int jg = lane / 16;         // K: 32-dim group; V: group of 4 tokens
    constexpr int T = FP8 ? kTileFp8 : kTileBf16;
    constexpr int NCH = T / 1024;     // 16-byte chunks per lane per tile

    const uint16_t* kbase = k_rows + row0 * row_elems;
    const uint16_t* vbase = v_rows + row0 * row_elems;
    // Rows of one head -> registers: each load instruction reads 4 whole
    // 256-byte rows (each byte once); tokens past the prompt become zeros.
    const auto load_head = [&](u32x4 (&kw)[4], u32x4 (&vw)[4], int g) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int piece = lane + 64 * k;
            const int r = piece / 16, c = piece % 16;
            const size_t off = static_cast<size_t>(r) * row_elems + static_cast<size_t>(g) * kDim + 8 * c;
            kw[k] = r < n ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + off))
                          : u32x4{0u, 0u, 0u, 0u};
            vw[k] = r < n ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + off))
                          : u32x4{0u, 0u, 0u, 0u};
        }
    };
    const auto stage = [&](const u32x4 (&w)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int piece = lane + 64 * k;
            *reinterpret_cast<u32x4*>(&sx[piece / 16][8 * (piece % 16)]) = w[k];
        }
        wave_lds_sync();
    };

    u32x4 kw[4], vw[4];
    load_head(kw, vw, wave);
    for (int g = wave; g < hkv; g += kIngestWaves) {
        const size_t tile = static_cast<size_t>(page) * hkv + g;
        uint8_t* kt = k_pool + tile * T + 16 * lane;
        uint8_t* vt = v_pool + tile * T + 16 * lane;
        // the next head's rows are in flight while this one is encoded
        u32x4 kn[4], vn[4];
        const bool more = g + kIngestWaves < hkv;        // wave-uniform
        if (more) load_head(kn, vn, g + kIngestWaves);
        // ---- K: lane holds token m, dims 32 jg + (16 h | 8 h) ..
        stage(kw);
        if constexpr (FP8) {
            const float ks = k_scale[g];
            const float kinv = 1.0f / ks;
            const auto encode_k = [&](auto recip) __attribute__((always_inline)) {
                constexpr bool R = decltype(recip)::value;
#pragma unroll
                for (int h = 0; h < NCH; ++h) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(&sx[m][32 * jg + 16 * h]);
                    const u32x4 b2 = *reinterpret_cast<const u32x4*>(&sx[m][32 * jg + 16 * h + 8]);
                    const uint32_t w[8] = {a[0], a[1], a[2], a[3], b2[0], b2[1], b2[2], b2[3]};
                    uint32_t c[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t lo = w[2 * e], hi = w[2 * e + 1];
                        c[e] = quant4_e4m3<R>(__uint_as_float(lo << 16), __uint_as_float(lo & 0xFFFF0000u),
                                              __uint_as_float(hi << 16), __uint_as_float(hi & 0xFFFF0000u),
                                              ks, kinv);
                    }
                    store_stream(kt + 1024 * h, u32x4{c[0], c[1], c[2], c[3]});
                }
            };
            // one uniform branch per head: the scale is the wave's, the range is voted on
            if (recip_quotient_ok(ks) && wave_recip_range(kw)) encode_k(std::true_type{});
            else encode_k(std::false_type{});
        } else {
#pragma unroll
            for (int h = 0; h < NCH; ++h)
                store_stream(kt + 1024 * h, *reinterpret_cast<const u32x4*>(&sx[m][32 * jg + 8 * h]));
        }
        wave_lds_sync();                                 // K reads done before V overwrites
        // ---- V: lane holds dim m of each 16-dim chunk, tokens 4 jg .. 4 jg + 3
        stage(vw);
        if constexpr (FP8) {
            const float vs = v_scale[g];
            const float vinv = 1.0f / vs;
            const auto encode_v = [&](auto recip) __attribute__((always_inline)) {
                constexpr bool R = decltype(recip)::value;
#pragma unroll
                for (int h = 0; h < NCH; ++h) {
                    uint32_t c[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {           // dword e: dim 64 h + 16 e + m
                        const int d = 64 * h + 16 * e + m;
                        float x[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) x[r] = bf16_bits_to_float(sx[4 * jg + r][d]);
                        c[e] = quant4_e4m3<R>(x[0], x[1], x[2], x[3], vs, vinv);
                    }
                    store_stream(vt + 1024 * h, u32x4{c[0], c[1], c[2], c[3]});
                }
            };
            if (recip_quotient_ok(vs) && wave_recip_range(vw)) encode_v(std::true_type{});
            else encode_v(std::false_type{});
        } else {
#pragma unroll
            for (int h = 0; h < NCH; ++h) {
                uint32_t c[4];
#pragma unroll
                for (int e = 0; e < 2; ++e) {               // half e: dim 32 h + 16 e + m
                    const int d = 32 * h + 16 * e + m;
                    uint32_t hv[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) hv[r] = sx[4 * jg + r][d];
                    c[2 * e] = hv[0] | (hv[1] << 16);
                    c[2 * e + 1] = hv[2] | (hv[3] << 16);
                }
                store_stream(vt + 1024 * h, u32x4{c[0], c[1], c[2], c[3]});
            }
        }
        wave_lds_sync();                                 // V reads done before the next head
        if (more) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                kw[k] = kn[k];
                vw[k] = vn[k];
            }
        }
    }
}

// Grid-stride over the (request, page) items, so any batch x max_pages fits
// a launch (most items of short prompts exit at once); the LDS blocks are
// per wavefront and every head ends with its reads complete, so items follow
// one another without a workgroup barrier.
constexpr int64_t kIngestMaxWgs = 65536;

template <bool FP8>
__global__ __launch_bounds__(kIngestWaves * 64) void ingest_kernel(
    const uint16_t* __restrict__ k_rows, const uint16_t* __restrict__ v_rows,
    int64_t n_rows, const int32_t* __restrict__ row_start, const int32_t* __restrict__ seq_lens,
    int32_t batch, int32_t max_seq_len, int32_t max_pages, const int32_t* __restrict__ block_table,
    int32_t bt_stride, const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool, int32_t num_pages, int32_t hkv,
    const uint8_t* __restrict__ abort) {
    __shared__ uint16_t sx_all[kIngestWaves][kPage][kVRowHalves];
    const int64_t n_items = static_cast<int64_t>(batch) * max_pages;
    for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x)
        ingest_page<FP8>(static_cast<int>(item / max_pages), static_cast<int>(item % max_pages),
                         k_rows, v_rows, n_rows, row_start, seq_lens, max_seq_len, block_table,
                         bt_stride, k_scale, v_scale, k_pool, v_pool, num_pages, hkv, abort,
                         sx_all[threadIdx.x / 64]);
}

hipError_t launch_amax(const uint16_t* x, int64_t n_rows, int32_t hkv, float* amax_inout,
                       hipStream_t stream) {
    const int64_t n_vec = n_rows * hkv * (kDim / 8);
    if (n_vec == 0) return hipSuccess;
    int64_t wgs = (n_vec + 4 * kAmaxThreads - 1) / (4 * kAmaxThreads);
    wgs = wgs < 2048 ? wgs : 2048;                // measured best of 1024 .. 16384
    wgs = (wgs + hkv - 1) / hkv * hkv;            // stride a multiple of 16 * hkv
    hipLaunchKernelGGL(amax_kernel, dim3(static_cast<uint32_t>(wgs)), dim3(kAmaxThreads), 0,
                       stream, reinterpret_cast<const u32x4*>(x), n_vec, hkv,
                       reinterpret_cast<uint32_t*>(amax_inout));
    return hipGetLastError();
}

hipError_t launch_scales(const float* amax, int32_t n, float* out, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const int wgs = (n + 255) / 256 < 64 ? (n + 255) / 256 : 64;
    hipLaunchKernelGGL(scales_kernel, dim3(wgs), dim3(256), 0, stream, amax, n, out);
    return hipGetLastError();
}

hipError_t launch_ingest(bool fp8, const uint16_t* k_rows, const uint16_t* v_rows,
                         int64_t n_rows, const int32_t* row_start, const int32_t* seq_lens, int32_t batch,
                         int32_t max_seq_len, const int32_t* block_table, int32_t bt_stride,
                         const float* k_scale, const float* v_scale, void* k_pool, void* v_pool,
                         int32_t num_pages, int32_t num_kv_heads, const uint8_t* abort,
                         hipStream_t stream) {
    const int32_t max_pages = (max_seq_len + kPage - 1) / kPage;
    if (batch == 0 || max_pages == 0) return hipSuccess;
    const dim3 grid(static_cast<uint32_t>(
        std::min<int64_t>(static_cast<int64_t>(batch) * max_pages, kIngestMaxWgs)));
    if (fp8) {
        hipLaunchKernelGGL(ingest_kernel<true>, grid, dim3(kIngestWaves * 64), 0, stream, k_rows,
                           v_rows, n_rows, row_start, seq_lens, batch, max_seq_len, max_pages, block_table,
                           bt_stride, k_scale, v_scale, static_cast<uint8_t*>(k_pool),
                           static_cast<uint8_t*>(v_pool), num_pages, num_kv_heads, abort);
    } else {
        hipLaunchKernelGGL(ingest_kernel<false>, grid, dim3(kIngestWaves * 64), 0, stream, k_rows,
                           v_rows, n_rows, row_start, seq_lens, batch, max_seq_len, max_pages, block_table,
                           bt_stride, nullptr, nullptr, static_cast<uint8_t*>(k_pool),
                           static_cast<uint8_t*>(v_pool), num_pages, num_kv_heads, abort);
    }
    return hipGetLastError();
}

}  // namespace kvfp8
