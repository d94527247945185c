// Weight-only quantized decode GEMV: y[m][n] += sum_k x[m][k] * q[n][k] * s[n][k / 128]
// with INT4 or FP8 e4m3 weight codes q and one fp32 scale per (row, 128-input
// group), bf16 activations x. Decode streams the weights from HBM for every
// token, so fewer weight bytes give each token sooner (remio.ai/it "Il serving
// di modelli più piccoli di Cloudflare riduce la memoria, ma la sicurezza
// diventa la prova decisiva", section "La compressione dei pesi GLM modifica
// il compromesso tra le fasi"); the codes are expanded before the product.
//
//  * packed layout (documented in kvfp8.h): block (nt, g) = rows 16 nt ..
//    16 nt + 15, inputs 128 g .. 128 g + 127; lane l of a wavefront owns the
//    16-byte chunk(s) at 16 l (+ 1 KiB) holding exactly its weight operands
//    of the four 16x16x32 bf16 MFMAs over the group (row l % 16, inputs
//    32 c + 8 (l / 16) + 0..7 of slice c), so each load is a coalesced 1 KiB;
//  * the activations are the MFMA's A operand (tokens down the rows) and the
//    weights its B operand, so a lane's four results are four tokens of one
//    weight row and the 16 lanes of a token add to 16 consecutive outputs
//    (one 64-byte line per atomic instruction and token group);
//  * integer codes (|q| <= 7) are sign-magnitude fields placed so that one
//    mask (values 0..3) or a rotate and a mask (values 4..7) leaves, in each
//    byte, an e4m3 subnormal of q * 2^-9; the hardware decode with scale 2^9
//    then gives q in bf16 exactly. e4m3 codes go through the decode alone;
//    the MFMA sums one group in fp32 and the group's row scale multiplies
//    that partial (the products themselves are exact);
//  * grid: a workgroup = 4 wavefronts = 4 consecutive 16-row tiles over one
//    range of input groups; ranges are split so the grid fills the chip, and
//    partial sums are added to y with hardware fp32 atomics (y must hold
//    zeros or a bias on entry);
//  * 1 .. 4 tokens (wq_gemv_small_kernel): the range's activations are staged
//    in LDS once, then each wavefront streams its codes through a 3-deep
//    register pipeline with no further barrier;
//  * 5 .. 64 tokens (wq_gemv_kernel): the activations pass through LDS in
//    double-buffered chunks loaded by the whole workgroup, each chunk's codes
//    one chunk ahead in registers.
#include <algorithm>

#include "kv_device.h"
#include "kv_launch.h"

namespace kvfp8 {

constexpr int kWGroup = 128;       // inputs per scale group
constexpr int kGemvWaves = 4;

// ---------------------------------------------------------------------------
// quantize + pack
// ---------------------------------------------------------------------------
// One wavefront per (16-row tile, group): lane (r = l % 16, j = l / 16) holds
// the 32 values of row r at inputs 32 c + 8 j + i (c, i < 8 | 4); the group's
// amax of row r is reduced over the 4 lanes r, r + 16, r + 32, r + 48.
template <bool INT4>
__global__ __launch_bounds__(256) void wq_pack_kernel(const uint16_t* __restrict__ w, int32_t n,
                                                      int32_t k, uint8_t* __restrict__ packed,
                                                      float* __restrict__ scales) {
    const int groups = k / kWGroup;
    const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
    if (item >= static_cast<int64_t>(n / 16) * groups) return;
    const int nt = static_cast<int>(item / groups);
    const int g = static_cast<int>(item % groups);
    const int lane = threadIdx.x % 64;
    const int r = lane % 16, j = lane / 16;
    const uint16_t* row = w + static_cast<size_t>(16 * nt + r) * k + kWGroup * g + 8 * j;
    u32x4 raw[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) raw[c] = *reinterpret_cast<const u32x4*>(row + 32 * c);
    uint32_t amax = 0;                                       // bf16 magnitude bits
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            amax = max(amax, raw[c][e] & 0x7FFFu);
            amax = max(amax, (raw[c][e] >> 16) & 0x7FFFu);
        }
    amax = max(amax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(amax), 16)));
    amax = max(amax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(amax), 32)));
    const float a = __uint_as_float(amax << 16);
    const float s = a > 0.0f ? a / (INT4 ? 7.0f : 448.0f) : 1.0f;
    const size_t blk = static_cast<size_t>(nt) * groups + g;
    if (j == 0) scales[blk * 16 + r] = s;
    if constexpr (INT4) {
        uint32_t d[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t bits = (raw[c][i / 2] >> (16 * (i % 2))) & 0xFFFFu;
                // round-to-odd quotient, then half-to-even to an integer: exact (24 >= 4 + 2);
                // |w / s| <= amax / fp32(amax / 7) < 7.5, so the clamp to [-7, 7] changes
                // nothing and three magnitude bits suffice
                const float qf = rintf(div_round_odd(bf16_bits_to_float(bits), s));
                const float qc = fminf(fmaxf(qf, -7.0f), 7.0f);
                const uint32_t mag = static_cast<uint32_t>(fabsf(qc));
                const uint32_t neg = qc < 0.0f ? 1u : 0u;
                const int j = i % 4;
                if (i < 4)      // byte j: magnitude in bits 0..2, sign in bit 7
                    word |= (mag << (8 * j)) | (neg << (8 * j + 7));
                else            // magnitude in bits 4..6 of byte j, sign in bit 3 of byte j + 1 (mod 4)
                    word |= (mag << (8 * j + 4)) | (neg << (8 * ((j + 1) % 4) + 3));
            }
            d[c] = word;
        }
        *reinterpret_cast<u32x4*>(packed + blk * 1024 + 16 * lane) = u32x4{d[0], d[1], d[2], d[3]};
    } else {
        uint32_t d[8];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t lo = raw[c][2 * h], hi = raw[c][2 * h + 1];
                d[2 * c + h] = encode4_e4m3(div_round_odd(bf16_bits_to_float(lo & 0xFFFF), s),
                                            div_round_odd(bf16_bits_to_float(lo >> 16), s),
                                            div_round_odd(bf16_bits_to_float(hi & 0xFFFF), s),
                                            div_round_odd(bf16_bits_to_float(hi >> 16), s));
            }
        // chunk 0 (at 16 l) holds slices 0, 1; chunk 1 (at 1024 + 16 l) slices 2, 3
        uint8_t* base = packed + blk * 2048 + 16 * lane;
        *reinterpret_cast<u32x4*>(base) = u32x4{d[0], d[1], d[2], d[3]};
        *reinterpret_cast<u32x4*>(base + 1024) = u32x4{d[4], d[5], d[6], d[7]};
    }
}

// ---------------------------------------------------------------------------
// GEMV
// ---------------------------------------------------------------------------
// One packed dword of 8 INT4 codes -> 8 bf16, exactly. Value i < 4 has its
// magnitude in bits 0..2 and its sign in bit 7 of byte i, so w & 0x87878787 is
// four e4m3 subnormals (+-|q| * 2^-9); value i + 4 has its magnitude in bits
// 4..6 of byte i and its sign in bit 3 of byte i + 1 (mod 4), so a rotate
// right by 4 and the same mask give the other four. The hardware decode with
// scale 2^9 returns q: ~0.9 VALU instructions per weight.
__device__ __forceinline__ bf16x8 int4x8_to_bf16(uint32_t w) {
    const uint32_t lo = w & 0x87878787u;                                  // values 0..3
    const uint32_t hi = __builtin_amdgcn_alignbit(w, w, 4) & 0x87878787u;  // values 4..7
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, false);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, true);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, false);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, true);
    return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo_w, uint32_t hi_w) {
    bf16x2 p0, p1, p2, p3;
    decode4_bf16(lo_w, p0, p1);
    decode4_bf16(hi_w, p2, p3);
    return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Groups of inputs per LDS chunk of activations, by m-tile count: the chunk
// (MT * 16 rows x CG * 128 inputs, double-buffered) stays within ~68 KiB.
// Chunk and grid sizes (measured on the decode layer shapes): with one m-tile
// (<= 16 tokens) short chunks and many workgroups keep the most weight bytes
// in flight; with more tokens fewer splits of the inputs cut the re-staged
// activations and the atomic adds. Two groups per chunk with two m-tiles
// (4 took 8% longer at 24-32 tokens); one with four m-tiles of INT4 weights
// (6% faster than 2 at 64 tokens, while FP8 weights were 10% slower with it).
#ifndef KVFP8_GEMV_CG1
#define KVFP8_GEMV_CG1 2          // groups per chunk with one m-tile
#endif
#ifndef KVFP8_GEMV_TARGET_WGS1
#define KVFP8_GEMV_TARGET_WGS1 2048   // up to 4 tokens (small-batch kernel)
#endif
#ifndef KVFP8_GEMV_TARGET_WGS
#define KVFP8_GEMV_TARGET_WGS 768     // 5 .. 16 tokens
#endif
#ifndef KVFP8_GEMV_TARGET_WGS3
#define KVFP8_GEMV_TARGET_WGS3 512    // more than 16 tokens
#endif
template <bool INT4, int MT>
struct GemvChunk {
    static constexpr int CG = MT == 1 ? KVFP8_GEMV_CG1 : (MT == 4 && INT4 ? 1 : 2);
    static constexpr int ROW = CG * kWGroup + 8;      // halves per LDS row (16-byte pad)
    static constexpr int PIECES = MT * 16 * CG * 16;  // 16-byte pieces per chunk
    static_assert(PIECES % (kGemvWaves * 64) == 0, "pieces per thread");
    static constexpr int PER_THREAD = PIECES / (kGemvWaves * 64);
};

template <bool INT4>
struct GroupCodes {
    u32x4 w[INT4 ? 1 : 2];
};

template <bool INT4, int MT>
__global__ __launch_bounds__(kGemvWaves * 64) void wq_gemv_kernel(
    const uint16_t* __restrict__ x, int32_t m_rows, const uint8_t* __restrict__ packed,
    const float* __restrict__ scales, int32_t n, int32_t k, float* __restrict__ y,
    int32_t groups_per_wg) {
    using C = GemvChunk<INT4, MT>;
    constexpr int CG = C::CG;
    __shared__ uint16_t xs[2][MT * 16][C::ROW];

    const int groups = k / kWGroup;
    const int n_tiles = n / 16;
    const int n_groups_rows = (n_tiles + kGemvWaves - 1) / kGemvWaves;   // 64-row groups
    const int wg_row = blockIdx.x % n_groups_rows;
    const int wg_k = blockIdx.x / n_groups_rows;
    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    const int nt = wg_row * kGemvWaves + wave;
    // a wave past the last tile still joins the chunk loads and barriers
    const bool active = nt < n_tiles;
    const int g0 = wg_k * groups_per_wg;
    const int g1 = min(groups, g0 + groups_per_wg);
    const int n_chunks = (g1 - g0 + CG - 1) / CG;
    const int col = lane % 16;          // A: token within the m-tile; B and result: weight row
    const int jg = lane / 16;           // A, B: input sub-slice; result: token group of 4

    // activation chunk ci -> registers (zeros past the rows or groups), then LDS
    u32x4 xr[C::PER_THREAD];
    const auto load_x = [&](int ci) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < C::PER_THREAD; ++u) {
            const int p = threadIdx.x + kGemvWaves * 64 * u;
            const int row = p / (CG * 16), c8 = p % (CG * 16);
            const int g = g0 + ci * CG + c8 / 16;
            xr[u] = (row < m_rows && g < g1)
                        ? *reinterpret_cast<const u32x4*>(x + static_cast<size_t>(row) * k +
                                                          static_cast<size_t>(kWGroup) * (g0 + ci * CG) + 8 * c8)
                        : u32x4{0u, 0u, 0u, 0u};
        }
    };
    const auto store_x = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < C::PER_THREAD; ++u) {
            const int p = threadIdx.x + kGemvWaves * 64 * u;
            const int row = p / (CG * 16), c8 = p % (CG * 16);
            *reinterpret_cast<u32x4*>(&xs[buf][row][8 * c8]) = xr[u];
        }
    };
    // codes and scales of chunk ci (groups past g1 are not loaded)
    GroupCodes<INT4> wc[CG];
    float sc[CG];
    const auto load_w = [&](int ci, GroupCodes<INT4> (&w)[CG], float (&s)[CG]) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < CG; ++q) {
            const int g = g0 + ci * CG + q;
            if (active && g < g1) {
                const size_t blk = static_cast<size_t>(nt) * groups + g;
                if constexpr (INT4) {
                    w[q].w[0] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4*>(packed + blk * 1024 + 16 * lane));
                } else {
                    w[q].w[0] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4*>(packed + blk * 2048 + 16 * lane));
                    w[q].w[1] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4*>(packed + blk * 2048 + 1024 + 16 * lane));
                }
                s[q] = scales[blk * 16 + col];
            }
        }
    };

    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (n_chunks > 0) {
        load_x(0);
        load_w(0, wc, sc);
        store_x(0);
    }
    __syncthreads();
    for (int ci = 0; ci < n_chunks; ++ci) {
        const int buf = ci & 1;
        const bool more = ci + 1 < n_chunks;                  // uniform over the workgroup
        GroupCodes<INT4> wn[CG];
        float sn[CG];
        if (more) {                                           // next chunk in flight
            load_x(ci + 1);
            load_w(ci + 1, wn, sn);
        }
        if (active) {
#pragma unroll
            for (int q = 0; q < CG; ++q) {
                if (g0 + ci * CG + q >= g1) break;            // uniform
                bf16x8 A[4];
                if constexpr (INT4) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) A[c] = int4x8_to_bf16(wc[q].w[0][c]);
                } else {
                    A[0] = e4m3x8_to_bf16(wc[q].w[0][0], wc[q].w[0][1]);
                    A[1] = e4m3x8_to_bf16(wc[q].w[0][2], wc[q].w[0][3]);
                    A[2] = e4m3x8_to_bf16(wc[q].w[1][0], wc[q].w[1][1]);
                    A[3] = e4m3x8_to_bf16(wc[q].w[1][2], wc[q].w[1][3]);
                }
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const u32x4 xb = *reinterpret_cast<const u32x4*>(
                            &xs[buf][16 * t + col][kWGroup * q + 32 * c + 8 * jg]);
                        part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, xb), A[c], part, 0, 0, 0);
                    }
                    acc[t] += sc[q] * part;     // column col is weight row 16 nt + col
                }
            }
        }
        if (more) {
            store_x(buf ^ 1);                  // the other buffer: last read before the barrier
#pragma unroll
            for (int q = 0; q < CG; ++q) {
                wc[q] = wn[q];
                sc[q] = sn[q];
            }
        }
        __syncthreads();
    }
    if (!active) return;
    // result layout: lane holds tokens 16 t + 4 jg + i of weight row 16 nt + col, so
    // the 16 lanes of one jg add to 16 consecutive outputs (one 64-byte line)
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * t + 4 * jg + i;
            if (m < m_rows) unsafeAtomicAdd(y + static_cast<size_t>(m) * n + 16 * nt + col, acc[t][i]);
        }
    }
}

// ---------------------------------------------------------------------------
// GEMV for 1 .. 4 tokens: no per-chunk barrier. The workgroup stages the
// activations of its whole input range (real rows only; m_rows x ng x 256 B
// of dynamic LDS) once, then every wavefront streams its tile's codes and
// scales through a 3-deep register pipeline while it reads its activation
// operands from LDS (a separate counter from the code loads, so the waits for
// the codes never wait on activations). Operand rows past the real tokens
// read token 0: their results are discarded, so no zero rows are stored.
// ---------------------------------------------------------------------------
// Up to 4 tokens (measured: from 5 tokens on the chunked kernel with 768
// workgroups is faster, at 8 tokens 58 against 68 us per INT4 layer).
#ifndef KVFP8_GEMV_SMALL_ROWS
#define KVFP8_GEMV_SMALL_ROWS 4
#endif
constexpr int kSmallMaxRows = KVFP8_GEMV_SMALL_ROWS;
// input groups per range whose activations are staged whole (4 rows x 16
// groups: 16.5 KiB of LDS)
__host__ __device__ constexpr int small_max_groups(int m_rows) { return m_rows <= 8 ? 16 : 8; }

template <bool INT4>
struct GroupTile {
    u32x4 w[INT4 ? 1 : 2];
    float s;                       // scale of weight row 16 nt + col
};

template <bool INT4>
__global__ __launch_bounds__(kGemvWaves * 64) __attribute__((amdgpu_waves_per_eu(4, 8)))
void wq_gemv_small_kernel(const uint16_t* __restrict__ x, int32_t m_rows,
                          const uint8_t* __restrict__ packed, const float* __restrict__ scales,
                          int32_t n, int32_t k, float* __restrict__ y, int32_t groups_per_wg) {
    extern __shared__ uint16_t xs_dyn[];
    constexpr int BLK = INT4 ? 1024 : 2048;                // code bytes per (tile, group)
    const int groups = k / kWGroup;
    const int n_tiles = n / 16;
    const int n_groups_rows = (n_tiles + kGemvWaves - 1) / kGemvWaves;
    const int wg_row = blockIdx.x % n_groups_rows;
    const int wg_k = blockIdx.x / n_groups_rows;
    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    const int nt = wg_row * kGemvWaves + wave;
    const int g0 = wg_k * groups_per_wg;
    const int ng = min(groups, g0 + groups_per_wg) - g0;  // 1 .. small_max_groups(m_rows)
    const int row_h = ng * kWGroup + 8;                    // halves per LDS row (16-byte pad)

    const int col = lane % 16;                             // A: token; B and result: weight row
    const int jg = lane / 16;                              // A, B: input sub-slice; result: token group
    const bool has_tile = nt < n_tiles;                    // uniform per wavefront
    // a wavefront past the last row tile keeps its pointers at tile 0 and loads nothing
    const size_t blk0 = static_cast<size_t>(has_tile ? nt : 0) * groups + g0;
    const uint8_t* cbase = packed + blk0 * BLK + 16 * lane;
    const float* sbase = scales + blk0 * 16 + col;

    const auto issue = [&](GroupTile<INT4>& t, int i) __attribute__((always_inline)) {
        const uint8_t* cp = cbase + static_cast<size_t>(i) * BLK;
        t.w[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(cp));
        if constexpr (!INT4) t.w[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(cp + 1024));
        t.s = sbase[static_cast<size_t>(i) * 16];
    };
    GroupTile<INT4> t0, t1, t2;
    const auto issue_first = [&]() __attribute__((always_inline)) {
        issue(t0, 0);
        if (ng > 1) issue(t1, 1);
        if (ng > 2) issue(t2, 2);
    };
    // The first three groups' codes do not depend on the activations. FP8 codes
    // are requested before the staging below, so their latency overlaps it
    // (2-4% faster at 1-4 tokens); INT4 codes measured ~3% slower that way at
    // one token, so they are requested after the barrier.
    constexpr bool kIssueBeforeStaging = !INT4;
    if (kIssueBeforeStaging && has_tile) issue_first();

    // activations of rows 0 .. m_rows - 1, inputs 128 g0 .. 128 (g0 + ng): 16-byte pieces
    const int per_row = ng * 16;
    for (int p = threadIdx.x; p < m_rows * per_row; p += kGemvWaves * 64) {
        const int row = p / per_row, c8 = p % per_row;
        *reinterpret_cast<u32x4*>(xs_dyn + row * row_h + 8 * c8) = *reinterpret_cast<const u32x4*>(
            x + static_cast<size_t>(row) * k + static_cast<size_t>(kWGroup) * g0 + 8 * c8);
    }
    __syncthreads();
    if (!has_tile) return;                                 // no barrier below
    if (!kIssueBeforeStaging) issue_first();

    const uint16_t* xb_base = xs_dyn + (col < m_rows ? col : 0) * row_h + 8 * jg;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const auto proc = [&](const GroupTile<INT4>& t, int i) __attribute__((always_inline)) {
        bf16x8 A[4];
        if constexpr (INT4) {
#pragma unroll
            for (int c = 0; c < 4; ++c) A[c] = int4x8_to_bf16(t.w[0][c]);
        } else {
            A[0] = e4m3x8_to_bf16(t.w[0][0], t.w[0][1]);
            A[1] = e4m3x8_to_bf16(t.w[0][2], t.w[0][3]);
            A[2] = e4m3x8_to_bf16(t.w[1][0], t.w[1][1]);
            A[3] = e4m3x8_to_bf16(t.w[1][2], t.w[1][3]);
        }
        f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4 xb = *reinterpret_cast<const u32x4*>(xb_base + kWGroup * i + 32 * c);
            part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xb), A[c],
                                                           part, 0, 0, 0);
        }
        acc += t.s * part;                 // column col is weight row 16 nt + col
    };
    // 3-deep pipeline (groups 0 .. 2 already requested): the steady-state loop
    // issues unconditionally (i + 5 < ng); the last 1 .. 5 groups are handled
    // with uniform conditions. INT4: each wavefront's scheduling priority
    // follows its progress through the range (3 in the first quarter, then
    // 2, 1, 0), so the workgroups resident on a CU finish closer together:
    // 2.4-3.3% off an INT4 layer at 1-4 tokens, while FP8 weights measured the
    // same or 0.3% slower with it (and the chunked kernel, ranked by chunk,
    // between 2% faster and 6% slower by token count and format).
    int i = 0;
    for (; i + 5 < ng; i += 3) {
        if constexpr (INT4) {
            const int quarter = (4 * i) / ng;
            if (quarter <= 0) __builtin_amdgcn_s_setprio(3);
            else if (quarter == 1) __builtin_amdgcn_s_setprio(2);
            else if (quarter == 2) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
        }
        proc(t0, i);
        issue(t0, i + 3);
        proc(t1, i + 1);
        issue(t1, i + 4);
        proc(t2, i + 2);
        issue(t2, i + 5);
    }
    proc(t0, i);
    if (i + 3 < ng) issue(t0, i + 3);
    if (i + 1 < ng) proc(t1, i + 1);
    if (i + 4 < ng) issue(t1, i + 4);
    if (i + 2 < ng) proc(t2, i + 2);
    if (i + 3 < ng) proc(t0, i + 3);
    if (i + 4 < ng) proc(t1, i + 4);

    // lane holds tokens 4 jg + r of weight row 16 nt + col
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = 4 * jg + r;
        if (m < m_rows) unsafeAtomicAdd(y + static_cast<size_t>(m) * n + 16 * nt + col, acc[r]);
    }
}

size_t wq_packed_bytes(int32_t n, int32_t k, bool int4) {
    return static_cast<size_t>(n) * k / (int4 ? 2 : 1);
}

hipError_t launch_wq_pack(bool int4, const uint16_t* w, int32_t n, int32_t k, uint8_t* packed,
                          float* scales, hipStream_t stream) {
    const int64_t items = static_cast<int64_t>(n / 16) * (k / kWGroup);
    if (items == 0) return hipSuccess;
    const dim3 grid(static_cast<uint32_t>((items + 3) / 4));
    if (int4)
        hipLaunchKernelGGL(wq_pack_kernel<true>, grid, dim3(256), 0, stream, w, n, k, packed, scales);
    else
        hipLaunchKernelGGL(wq_pack_kernel<false>, grid, dim3(256), 0, stream, w, n, k, packed, scales);
    return hipGetLastError();
}

// y += W x for m_rows <= 64 (callers split larger batches).
hipError_t launch_wq_gemv(bool int4, const uint16_t* x, int32_t m_rows, const uint8_t* packed,
                          const float* scales, int32_t n, int32_t k, float* y,
                          hipStream_t stream) {
    if (m_rows == 0 || n == 0 || k == 0) return hipSuccess;
    const int groups = k / kWGroup;
    const int64_t row_groups = (n / 16 + kGemvWaves - 1) / kGemvWaves;
    // split the input groups so the grid holds ~4 workgroups per CU, at least 2 groups each
    const int mt = (m_rows + 15) / 16;
    const int64_t target = m_rows <= kSmallMaxRows ? KVFP8_GEMV_TARGET_WGS1
                           : m_rows <= 16 ? KVFP8_GEMV_TARGET_WGS : KVFP8_GEMV_TARGET_WGS3;
    int64_t splits = (target + row_groups - 1) / row_groups;
    splits = std::min<int64_t>(splits, std::max(1, groups / 2));
    const int per = static_cast<int>((groups + splits - 1) / splits);
    splits = (groups + per - 1) / per;
    if (m_rows <= kSmallMaxRows) {
        // at most small_max_groups input groups per range (the activations of a
        // range are staged whole)
        const int max_g = small_max_groups(m_rows);
        int64_t sp = std::max<int64_t>(splits, (groups + max_g - 1) / max_g);
        const int per_s = static_cast<int>((groups + sp - 1) / sp);
        sp = (groups + per_s - 1) / per_s;
        const dim3 grid_s(static_cast<uint32_t>(row_groups * sp));
        const size_t lds = static_cast<size_t>(m_rows) * (per_s * kWGroup + 8) * sizeof(uint16_t);
        if (int4)
            hipLaunchKernelGGL(wq_gemv_small_kernel<true>, grid_s, dim3(kGemvWaves * 64), lds, stream,
                               x, m_rows, packed, scales, n, k, y, per_s);
        else
            hipLaunchKernelGGL(wq_gemv_small_kernel<false>, grid_s, dim3(kGemvWaves * 64), lds, stream,
                               x, m_rows, packed, scales, n, k, y, per_s);
        return hipGetLastError();
    }
    const dim3 grid(static_cast<uint32_t>(row_groups * splits));
#define KVFP8_GEMV(I4, MTV)                                                                     \
    hipLaunchKernelGGL((wq_gemv_kernel<I4, MTV>), grid, dim3(kGemvWaves * 64), 0, stream, x,    \
                       m_rows, packed, scales, n, k, y, per)
    if (int4) {
        if (mt == 1) KVFP8_GEMV(true, 1); else if (mt == 2) KVFP8_GEMV(true, 2);
        else if (mt == 3) KVFP8_GEMV(true, 3); else KVFP8_GEMV(true, 4);
    } else {
        if (mt == 1) KVFP8_GEMV(false, 1); else if (mt == 2) KVFP8_GEMV(false, 2);
        else if (mt == 3) KVFP8_GEMV(false, 3); else KVFP8_GEMV(false, 4);
    }
#undef KVFP8_GEMV
    return hipGetLastError();
}

}  // namespace kvfp8
