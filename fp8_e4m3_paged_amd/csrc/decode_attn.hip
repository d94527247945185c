// Split-K paged decode attention over an FP8 e4m3 (or BF16) KV cache.
//
// What it computes is standard softmax attention of one decode token per
// query head over the request's cached tokens; the FP8 values are converted
// when the kernel reads them (remio.ai/it "Il serving di modelli più piccoli
// di Cloudflare ...", section "Perché le cache più piccole di Cloudflare
// battono la velocità pura": the conversion work sits in the attention
// kernel's reads). Decode is memory-bound (same page, same section), so the
// kernel is built to stream the cache at HBM speed:
//
//  * one 256-thread workgroup per (partition p, request b, KV head g); its
//    4 wavefronts take the partition's page *pairs* round-robin and keep the
//    next pair's loads in flight while computing the current one;
//  * a (page, head) tile is 2 KiB (FP8) and is read with 16-byte-per-lane
//    loads that cover it contiguously; the tile layout puts every byte in
//    the lane that needs it for the matrix-core step, so nothing is staged;
//  * QK^T of the GQA group runs on v_mfma_f32_16x16x32_bf16: A = 16 tokens x
//    32 dims of K (e4m3 -> bf16 is exact), B = 32 dims x 16 query columns of
//    Q (bf16, exact); the G <= 16 query heads of the group fill the columns;
//  * the online softmax works on the 16x16 score tile in the accumulator
//    layout (lane = query column, 4 token rows per lane): max and sum are a
//    4-value in-lane reduction plus two cross-lane xor steps;
//  * P.V runs on v_mfma_f32_16x16x32_f16 over the pair's 32 tokens: A = V^T
//    (e4m3 -> f16 is exact), B = P^T taken straight from the score registers
//    and rounded to f16 (nearest-even). BF16 caches use the bf16 instruction
//    with P split into a bf16 high and low part (two products) instead;
//  * the 4 (or 8) wavefronts merge their (max, sum, output) in LDS; with one
//    partition the workgroup writes the final output, otherwise a partial
//    that reduce_partials_kernel combines across partitions.
#include <algorithm>

#include "kv_device.h"
#include "kv_launch.h"

namespace kvfp8 {

constexpr int kWaves = 4;                      // wavefronts per workgroup (wave mode, shared)
constexpr int kWavesWide = 8;                  // shared mode when the grid fills one per CU
constexpr int kAccStride = kDim + 4;           // padded LDS row (floats)
constexpr float kLog2e = 1.4426950408889634f;
// Partitions up to this many tokens may run in the persistent kernel.
constexpr int kWaveModeMaxTokens = 2048;
// FP8 register pipeline depth of the shared kernel (page pairs in flight + 1);
// the persistent kernel keeps 3 (its fused form has no registers for a 4th).
#ifndef KVFP8_SHARED_DEPTH
#define KVFP8_SHARED_DEPTH 3
#endif
constexpr int kSharedDepth = KVFP8_SHARED_DEPTH;

// Raw registers of one page pair: K and V tiles of pages a and b.
template <bool FP8>
struct PairTiles {
    static constexpr int N = FP8 ? 2 : 4;     // 16-byte loads per lane per tile
    u32x4 ka[N], kb[N], va[N], vb[N];
};

template <bool FP8>
__device__ __forceinline__ void load_pair(PairTiles<FP8>& r, const uint8_t* __restrict__ k_pool,
                                 const uint8_t* __restrict__ v_pool, size_t tile_a,
                                 size_t tile_b, int lane) {
    constexpr int T = FP8 ? kTileFp8 : kTileBf16;
    const uint8_t* ka = k_pool + tile_a * T + 16 * lane;
    const uint8_t* kb = k_pool + tile_b * T + 16 * lane;
    const uint8_t* va = v_pool + tile_a * T + 16 * lane;
    const uint8_t* vb = v_pool + tile_b * T + 16 * lane;
    // The cache is streamed once per step: non-temporal loads keep it from
    // displacing reusable lines in the caches.
#pragma unroll
    for (int h = 0; h < PairTiles<FP8>::N; ++h) {
        r.ka[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ka + 1024 * h));
        r.kb[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + 1024 * h));
        r.va[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(va + 1024 * h));
        r.vb[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + 1024 * h));
    }
}

// A operand of QK^T MFMA c for one page: slot i <- dim 32j + 8c + i, which is
// bytes 8(c%2)..+7 of the lane's load c/2 (FP8, decoded to bf16) or load c
// itself (BF16).
template <bool FP8>
__device__ __forceinline__ bf16x8 k_operand(const u32x4 (&k)[PairTiles<FP8>::N], int c) {
    if constexpr (FP8) {
        bf16x2 p0, p1, p2, p3;
        decode4_bf16(k[c / 2][2 * (c % 2)], p0, p1);
        decode4_bf16(k[c / 2][2 * (c % 2) + 1], p2, p3);
        return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    } else {
        return __builtin_bit_cast(bf16x8, k[c]);
    }
}

// S^T (16 tokens x 16 query columns) of pages a and b: two chains of 4 MFMAs
// over head_dim, interleaved so neither waits on its own previous result.
template <bool FP8>
__device__ __forceinline__ void qk_pair(const PairTiles<FP8>& t, const bf16x8 (&qop)[4], f32x4& sa,
                               f32x4& sb) {
    sa = f32x4{0.f, 0.f, 0.f, 0.f};
    sb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<FP8>(t.ka, c), qop[c], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<FP8>(t.kb, c), qop[c], sb, 0, 0, 0);
    }
}

// Zero the bytes of tokens >= valid in a lane's 4-token groups (FP8: 1 byte
// per token per dword; BF16: 2 bytes per token, two dwords per group).
__device__ __forceinline__ uint32_t token_mask_fp8(int valid) {
    return valid >= 4 ? 0xFFFFFFFFu : (valid <= 0 ? 0u : ((1u << (8 * valid)) - 1u));
}
__device__ __forceinline__ uint64_t token_mask_bf16(int valid) {
    return valid >= 4 ? ~0ull : (valid <= 0 ? 0ull : ((1ull << (16 * valid)) - 1ull));
}

// (Whole-vector updates only: element stores into these register arrays can
// push them out to scratch memory.)
template <bool FP8>
__device__ __forceinline__ void mask_v(u32x4 (&v)[PairTiles<FP8>::N], int valid) {
    if constexpr (FP8) {
        const uint32_t m = token_mask_fp8(valid);
        const u32x4 mm = {m, m, m, m};
#pragma unroll
        for (int h = 0; h < 2; ++h) v[h] = v[h] & mm;
    } else {
        const uint64_t m = token_mask_bf16(valid);
        const uint32_t lo = static_cast<uint32_t>(m), hi = static_cast<uint32_t>(m >> 32);
        const u32x4 mm = {lo, hi, lo, hi};
#pragma unroll
        for (int h = 0; h < 4; ++h) v[h] = v[h] & mm;
    }
}

// Running-max slack (log2 units): the reference max m_run only moves when a
// new score exceeds it by more than this, so most pairs skip the rescale of
// the output accumulators. Probabilities then stay <= 2^8, which f16 holds
// with full precision; the normaliser is built against the same reference.
constexpr float kMaxSlack = 8.0f;

// One page pair of the online softmax: raw scores of pages a and b (tokens
// tok_a .. tok_a + 31), the running max / sum update and the P.V accumulation.
// s_scale = sm_scale * k_scale * log2(e) >= 0 multiplies the raw q.k sums, so
// the max is taken on raw sums and the scale is folded into exp2's argument.
// Only the pair that crosses t_end needs masking. Control flow is
// wave-uniform (MFMA needs all lanes).
template <bool FP8>
__device__ __forceinline__ void process_pair(PairTiles<FP8>& cur, int tok_a, int t_end, int jgrp,
                                    float s_scale, const bf16x8 (&qop)[4], float& m_run,
                                    float& l_run, f32x4 (&acc_o)[8]) {
    const int tok_b = tok_a + kPage;
    const bool tail = tok_b + kPage > t_end;
    if (tail) {
        // Tokens past t_end (the tail of the last page, or a missing page b)
        // must not contribute: their V bytes are zeroed (the slots may hold
        // stale codes, NaN included) and their scores masked below.
        mask_v<FP8>(cur.va, t_end - (tok_a + 4 * jgrp));
        mask_v<FP8>(cur.vb, t_end - (tok_b + 4 * jgrp));
    }
    f32x4 sa, sb;
    qk_pair<FP8>(cur, qop, sa, sb);
    float s[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
    if (tail) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (tok_a + 4 * jgrp + r >= t_end) s[r] = -INFINITY;
            if (tok_b + 4 * jgrp + r >= t_end) s[4 + r] = -INFINITY;
        }
    }
    // This lane's 8 scores; only if one of them exceeds the reference by the
    // slack (always on the first pair, where m_run is -inf) does the wave take
    // the column max over the 4 lanes of each column and rescale.
    const float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                           fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7]))) * s_scale;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kMaxSlack) != 0) {
        float mcol = fmaxf(mx, __shfl_xor(mx, 16));
        mcol = fmaxf(mcol, __shfl_xor(mcol, 32));
        const float m_new = fmaxf(m_run, mcol);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);    // 0 when m_run = -inf
        l_run *= alpha;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc_o[c] *= alpha;
        m_run = m_new;
    }
    float pv[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) pv[r] = __builtin_amdgcn_exp2f(fmaf(s[r], s_scale, -m_run));
    if (tail) {
        // explicit zeros: with s_scale == 0 the masked -inf would give NaN
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (tok_a + 4 * jgrp + r >= t_end) pv[r] = 0.f;
            if (tok_b + 4 * jgrp + r >= t_end) pv[4 + r] = 0.f;
        }
    }
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) psum += pv[r];
    l_run += psum;

    if constexpr (FP8) {
        // B = P^T: slots 0..3 = page a tokens 4j..4j+3, 4..7 = page b.
        f16x8 P;
#pragma unroll
        for (int r = 0; r < 8; r += 2) {
            const f16x2 h2 = __builtin_convertvector((f32x2{pv[r], pv[r + 1]}), f16x2);
            P[r] = h2[0];
            P[r + 1] = h2[1];
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            // A = V^T: row = dim 16c + col, slots = tokens 4j..4j+3 of
            // page a then of page b (dword c%4 of load c/4).
            f16x2 a0, a1, b0, b1;
            decode4_f16(cur.va[c / 4][c % 4], a0, a1);
            decode4_f16(cur.vb[c / 4][c % 4], b0, b1);
            const f16x8 A = {a0[0], a0[1], a1[0], a1[1], b0[0], b0[1], b1[0], b1[1]};
            acc_o[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, P, acc_o[c], 0, 0, 0);
        }
    } else {
        // P = hi + lo, both bf16: hi = RNE(p), lo = RNE(p - hi).
        bf16x8 Ph, Pl;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const __bf16 h = static_cast<__bf16>(pv[r]);
            Ph[r] = h;
            Pl[r] = static_cast<__bf16>(pv[r] - static_cast<float>(h));
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const u32x4 w = {cur.va[c / 2][2 * (c % 2)], cur.va[c / 2][2 * (c % 2) + 1],
                             cur.vb[c / 2][2 * (c % 2)], cur.vb[c / 2][2 * (c % 2) + 1]};
            const bf16x8 A = __builtin_bit_cast(bf16x8, w);
            acc_o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Ph, acc_o[c], 0, 0, 0);
            acc_o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Pl, acc_o[c], 0, 0, 0);
        }
    }
}

// The new token's codes, computed by the lanes that hold its bytes once
// loaded. Lane (t, j) holds K dims 32j..32j+31 of token t; lane (m, j) holds
// V dim 16c + m of tokens 4j..4j+3 for every chunk c. K: the lane's 16-byte
// chunks of that slot (2 for FP8, 4 for BF16). V: the 8 values of dims
// 16c + m (FP8: 8 codes in 2 dwords; BF16: 8 halves in 4 dwords).
template <bool FP8>
struct NewToken {
    u32x4 k[PairTiles<FP8>::N];
    uint32_t v[FP8 ? 2 : 4];
};

// The bf16 inputs a lane needs for its part of the new token: K dims
// 32j..32j+31 (64 bytes) and V dims 16c + m, c = 0..7.
struct NewTokenRaw {
    u32x4 k[4];
    uint16_t v[8];
};

__device__ __forceinline__ void load_new_token(NewTokenRaw& r, int lane, const uint16_t* __restrict__ krow,
                                      const uint16_t* __restrict__ vrow) {
    const int m = lane % 16;
    const int j = lane / 16;
#pragma unroll
    for (int h = 0; h < 4; ++h) r.k[h] = *reinterpret_cast<const u32x4*>(krow + 32 * j + 8 * h);
#pragma unroll
    for (int c = 0; c < 8; ++c) r.v[c] = vrow[16 * c + m];
}

// Encode (same arithmetic as kv_append_quant) in registers only.
template <bool FP8>
__device__ __forceinline__ void encode_new_token(NewToken<FP8>& nt, const NewTokenRaw& r, float ks,
                                        float vs) {
    if constexpr (FP8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t c4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const u32x4 w = r.k[2 * h + e / 2];            // dims 32j + 16h + 4e ..
                const uint32_t lo = w[2 * (e % 2)], hi = w[2 * (e % 2) + 1];
                c4[e] = encode4_e4m3(div_round_odd(bf16_bits_to_float(lo & 0xFFFF), ks),
                                     div_round_odd(bf16_bits_to_float(lo >> 16), ks),
                                     div_round_odd(bf16_bits_to_float(hi & 0xFFFF), ks),
                                     div_round_odd(bf16_bits_to_float(hi >> 16), ks));
            }
            nt.k[h] = u32x4{c4[0], c4[1], c4[2], c4[3]};
        }
        float y[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) y[c] = div_round_odd(bf16_bits_to_float(r.v[c]), vs);
        nt.v[0] = encode4_e4m3(y[0], y[1], y[2], y[3]);
        nt.v[1] = encode4_e4m3(y[4], y[5], y[6], y[7]);
    } else {
#pragma unroll
        for (int h = 0; h < 4; ++h) nt.k[h] = r.k[h];
#pragma unroll
        for (int c = 0; c < 8; c += 2)
            nt.v[c / 2] = static_cast<uint32_t>(r.v[c]) | (static_cast<uint32_t>(r.v[c + 1]) << 16);
    }
}

// Store the new token's codes into its pool tiles for later steps (K: whole
// 16-byte chunks, which hold only this slot; V: single bytes / halves, so the
// other slots of the same dwords keep their bytes). Runs after the wave's
// last load so its stores cannot disturb the pipeline's wait counts.
template <bool FP8>
__device__ __forceinline__ void store_new_token(const NewToken<FP8>& nt, int slot, int lane,
                                       uint8_t* __restrict__ ktile, uint8_t* __restrict__ vtile) {
    const int m = lane % 16;
    const int j = lane / 16;
    if (m == slot) {
#pragma unroll
        for (int h = 0; h < PairTiles<FP8>::N; ++h)
            *reinterpret_cast<u32x4*>(ktile + 1024 * h + 16 * lane) = nt.k[h];
    }
    if (j == slot / 4) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            if constexpr (FP8) {
                vtile[off_v_fp8(slot, 16 * c + m)] = static_cast<uint8_t>(nt.v[c / 4] >> (8 * (c % 4)));
            } else {
                *reinterpret_cast<uint16_t*>(vtile + off_v_bf16(slot, 16 * c + m)) =
                    static_cast<uint16_t>(nt.v[c / 2] >> (16 * (c % 2)));
            }
        }
    }
}

// Overwrite the new token's slot in one page's K / V registers with its codes
// when `on` (the token is in this page). Value selects only, called for both
// pages of the pair: choosing between the two pages' arrays at run time would
// force them out of registers.
template <bool FP8>
__device__ __forceinline__ void apply_new_token(u32x4 (&K)[PairTiles<FP8>::N],
                                                u32x4 (&V)[PairTiles<FP8>::N],
                                                const NewToken<FP8>& nt, int slot, int lane,
                                                bool on) {
    const int m = lane % 16;
    const int j = lane / 16;
    const bool pk = on && m == slot;
#pragma unroll
    for (int h = 0; h < PairTiles<FP8>::N; ++h) K[h] = pk ? nt.k[h] : K[h];
    const bool pv = on && j == slot / 4;
    const int sel = slot % 4;
    if constexpr (FP8) {
        // load h holds chunks c = 4h..4h+3, one dword each, token byte sel
        const uint32_t keep = ~(0xFFu << (8 * sel));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4 w = V[h];
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = (w[e] & keep) | (((nt.v[h] >> (8 * e)) & 0xFFu) << (8 * sel));
            V[h] = pv ? u32x4{o[0], o[1], o[2], o[3]} : w;
        }
    } else {
        // load h holds chunks c = 2h, 2h+1: dwords 2(c%2) (tokens 0, 1) and
        // 2(c%2) + 1 (tokens 2, 3) of the 4-token group; half sel % 2
        const uint32_t keep = ~(0xFFFFu << (16 * (sel % 2)));
        const bool upper = sel >= 2;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const u32x4 w = V[h];
            uint32_t o[4] = {w[0], w[1], w[2], w[3]};
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const uint32_t val = (nt.v[h] >> (16 * cc)) & 0xFFFFu;   // chunk 2h + cc
                const uint32_t lo2 = (o[2 * cc] & keep) | (val << (16 * (sel % 2)));
                const uint32_t hi2 = (o[2 * cc + 1] & keep) | (val << (16 * (sel % 2)));
                o[2 * cc] = upper ? o[2 * cc] : lo2;
                o[2 * cc + 1] = upper ? hi2 : o[2 * cc + 1];
            }
            V[h] = pv ? u32x4{o[0], o[1], o[2], o[3]} : w;
        }
    }
}

// Software pipeline over a wavefront's n page pairs: register buffers rotate
// so that while one pair is processed the next ones are in flight (DEPTH - 1
// of them for FP8: two or three; one for BF16, whose tiles take twice the
// registers). Every load in the steady-state loop is unconditional (the index
// is clamped to the last pair), so each wait is a static partial vmcnt; the
// FP8 epilogue issues only the loads that are still needed.
// `proc_end` processes the pairs of the FP8 epilogue, which always include
// the wave's last pair (the only one the fused append ever patches), so the
// steady-state loop carries no patch logic.
//
// PRIO: the wave's scheduling priority follows its own progress through its
// pairs (3 in the first quarter, then 2, 1, 0). Two 4-wave workgroups share a
// CU; without it the one that started first finishes well before the other
// (a per-workgroup timing probe saw ~95-110 against up to ~175 us at 64
// requests), which then streams alone. Ranked by progress, the later one
// catches up and the CU stays loaded to the end: at 64 requests x ~8.7k
// tokens the launch went 180 -> 178 us (FP8) and 355 -> 350 us (BF16), and
// the persistent kernel (two 4-wave workgroups per CU, progress counted per
// piece) on 16 requests of up to 131k tokens 186-188 -> 184 us. With one
// 8-wave workgroup per CU (32 requests) it measured 0.5-1% slower, so the
// 8-wave instance does not use it.
__device__ __forceinline__ void progress_priority(int i, int n) {
    const int quarter = (4 * i) / n;                      // 0 <= i < n
    if (quarter <= 0) __builtin_amdgcn_s_setprio(3);
    else if (quarter == 1) __builtin_amdgcn_s_setprio(2);
    else if (quarter == 2) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

template <bool FP8, int DEPTH, bool PRIO, typename Issue, typename Proc, typename ProcEnd,
          typename Hook>
__device__ __forceinline__ void pipeline_pairs(int n, Issue&& issue, Proc&& proc, ProcEnd&& proc_end,
                                               Hook&& after_issue) {
    if (n <= 0) return;
    if constexpr (FP8 && DEPTH == 4) {
        PairTiles<FP8> t0, t1, t2, t3;
        issue(t0, 0);
        issue(t1, 1);
        issue(t2, 2);
        issue(t3, 3);
        after_issue();     // runs while the first tiles are in flight
        int i = 0;
        for (; i + 7 < n; i += 4) {
            if constexpr (PRIO) progress_priority(i, n);
            proc(t0, i);
            issue(t0, i + 4);
            proc(t1, i + 1);
            issue(t1, i + 5);
            proc(t2, i + 2);
            issue(t2, i + 6);
            proc(t3, i + 3);
            issue(t3, i + 7);
        }
        // 1..7 pairs left: t0..t3 hold pairs i .. i+3 (when they exist)
        proc_end(t0, i);
        if (i + 4 < n) issue(t0, i + 4);
        if (i + 1 < n) proc_end(t1, i + 1);
        if (i + 5 < n) issue(t1, i + 5);
        if (i + 2 < n) proc_end(t2, i + 2);
        if (i + 6 < n) issue(t2, i + 6);
        if (i + 3 < n) proc_end(t3, i + 3);
        if (i + 4 < n) proc_end(t0, i + 4);
        if (i + 5 < n) proc_end(t1, i + 5);
        if (i + 6 < n) proc_end(t2, i + 6);
    } else if constexpr (FP8) {
        static_assert(DEPTH == 3, "FP8 pipelines are 3 or 4 deep");
        PairTiles<FP8> t0, t1, t2;
        issue(t0, 0);
        issue(t1, 1);
        issue(t2, 2);
        after_issue();     // runs while the first tiles are in flight
        int i = 0;
        for (; i + 5 < n; i += 3) {
            if constexpr (PRIO) progress_priority(i, n);
            proc(t0, i);
            issue(t0, i + 3);
            proc(t1, i + 1);
            issue(t1, i + 4);
            proc(t2, i + 2);
            issue(t2, i + 5);
        }
        // 1..5 pairs left: t0, t1, t2 hold pairs i, i+1, i+2 (when they exist)
        proc_end(t0, i);
        if (i + 3 < n) issue(t0, i + 3);
        if (i + 1 < n) proc_end(t1, i + 1);
        if (i + 4 < n) issue(t1, i + 4);
        if (i + 2 < n) proc_end(t2, i + 2);
        if (i + 3 < n) proc_end(t0, i + 3);
        if (i + 4 < n) proc_end(t1, i + 4);
    } else {
        // BF16: no separate epilogue (its straight-line copies of the pair step
        // exceed the register file); past the end the clamped loads re-read
        // the wave's last pair.
        PairTiles<FP8> t0, t1;
        issue(t0, 0);
        issue(t1, 1);
        after_issue();
        for (int i = 0; i < n; i += 2) {
            if constexpr (PRIO) progress_priority(i, n);
            proc_end(t0, i);
            issue(t0, i + 2);
            if (i + 1 < n) proc_end(t1, i + 1);
            issue(t1, i + 3);
        }
    }
}

// B operand of QK^T for query heads q_row .. q_row + group - 1: column col =
// query head q_row + col, slots = dims 32*jgrp + 8c + i. Columns past the
// group stay zero.
__device__ __forceinline__ void load_q_operand(bf16x8 (&qop)[4], const uint16_t* __restrict__ q,
                                               size_t q_row, int group, int col, int jgrp) {
    if (col < group) {
        const u32x4* qp = reinterpret_cast<const u32x4*>(q + (q_row + col) * kDim + 32 * jgrp);
#pragma unroll
        for (int c = 0; c < 4; ++c) qop[c] = __builtin_bit_cast(bf16x8, qp[c]);
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) qop[c] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
}

// One wavefront's share of the partition [t_begin, t_end) of (b, g): page
// pairs first, first + stride, ... of the partition's npg pages, where page k
// of the partition is pool tile tile_of(k). Accumulates the online softmax
// into (m_run, l_run, acc_o).
// APPEND: the wavefront whose share holds the new token t = L - 1 loads its
// bf16 K/V row (k_row, v_row) before its first tile loads (so every wait
// count in the pipeline stays static), encodes it (same encoder as
// kv_append_quant) while those tiles are in flight, overwrites the token's
// slot in the pair's registers when it gets there, and stores the codes to
// the pool after its last load. Nothing in the launch reads those codes back
// from memory, so no fence or barrier is involved.
template <bool FP8, bool APPEND, int DEPTH, bool PRIO, typename TileOf>
__device__ __forceinline__ void stream_share(
    TileOf&& tile_of, uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool, int npg,
    int pg0, int first, int stride, int t_begin, int t_end, int L, int lane, int jgrp,
    float s_scale, const bf16x8 (&qop)[4], const uint16_t* __restrict__ k_row,
    const uint16_t* __restrict__ v_row, const float* __restrict__ ks_ptr,
    const float* __restrict__ vs_ptr, float& m_run, float& l_run, f32x4 (&acc_o)[8]) {
    const int npairs = (npg + 1) / 2;
    const int n_w = npairs > first ? (npairs - first + stride - 1) / stride : 0;
    const auto issue = [&](PairTiles<FP8>& t, int i) __attribute__((always_inline)) {
        const int pr = first + stride * min(i, n_w - 1);
        load_pair<FP8>(t, k_pool, v_pool, tile_of(2 * pr), tile_of(min(2 * pr + 1, npg - 1)),
                       lane);
    };
    const int t_new = L - 1;
    const int pr_new = (t_new / kPage - pg0) / 2;
    const bool owns_new = APPEND && t_new >= t_begin && t_new < t_end && pr_new >= first &&
                          (pr_new - first) % stride == 0;
    const bool new_in_b = ((t_new / kPage - pg0) % 2) == 1;
    NewTokenRaw raw;
    NewToken<FP8> nt;
    if constexpr (APPEND) {
        if (owns_new) load_new_token(raw, lane, k_row, v_row);
    }
    const auto prepare = [&]() __attribute__((always_inline)) {
        if constexpr (APPEND) {
            if (owns_new) encode_new_token<FP8>(nt, raw, FP8 ? *ks_ptr : 1.0f, FP8 ? *vs_ptr : 1.0f);
        }
    };
    const auto proc = [&](PairTiles<FP8>& t, int i) __attribute__((always_inline)) {
        process_pair<FP8>(t, (pg0 + 2 * (first + stride * i)) * kPage, t_end, jgrp, s_scale, qop,
                          m_run, l_run, acc_o);
    };
    const auto proc_end = [&](PairTiles<FP8>& t, int i) __attribute__((always_inline)) {
        const int pr = first + stride * i;
        if constexpr (APPEND) {
            if (owns_new && pr == pr_new) {                  // wave-uniform
                apply_new_token<FP8>(t.ka, t.va, nt, t_new % kPage, lane, !new_in_b);
                apply_new_token<FP8>(t.kb, t.vb, nt, t_new % kPage, lane, new_in_b);
            }
        }
        process_pair<FP8>(t, (pg0 + 2 * pr) * kPage, t_end, jgrp, s_scale, qop, m_run, l_run,
                          acc_o);
    };
    pipeline_pairs<FP8, DEPTH, PRIO>(n_w, issue, proc, proc_end, prepare);
    if constexpr (APPEND) {
        if (owns_new) {
            const size_t tile = tile_of(t_new / kPage - pg0);
            constexpr int T = FP8 ? kTileFp8 : kTileBf16;
            store_new_token<FP8>(nt, t_new % kPage, lane, k_pool + tile * T, v_pool + tile * T);
        }
    }
}

__device__ __forceinline__ bool request_ok(const int32_t* __restrict__ seq_lens,
                                           const uint8_t* __restrict__ abort, int b, int L,
                                           int32_t max_seq_len, int32_t bt_stride) {
    const bool aborted = abort != nullptr && abort[b] != 0;
    return !aborted && L >= 1 && L <= max_seq_len &&
           (static_cast<int64_t>(L) + kPage - 1) / kPage <= bt_stride;
}

// LDS floats of the wavefront merge: [NW][16] maxima, [NW][16] sums and
// [NW][group][kAccStride] unnormalised outputs.
__host__ __device__ constexpr int merge_floats(int nw, int group) {
    return 2 * nw * 16 + nw * group * kAccStride;
}

// Combine the online-softmax states (m, l, acc) of the NW wavefronts that
// shared one stretch of a (request, KV head) through LDS at `sm` (laid out as
// merge_floats says). For every query head qh of the group and every 4 dims d,
// store(qh, d, M, lt, o) receives the combined maximum M (log2 units), the
// normaliser lt and the unnormalised output o (weighted by 2^(m_w - M)).
// Starts with a barrier after the LDS writes; callers that write the area
// again afterwards must synchronise first.
template <int NW, typename Store>
__device__ __forceinline__ void merge_waves(float* sm, int wave, int lane, int group, float m_run,
                                            float l_tot, const f32x4 (&acc_o)[8], Store&& store) {
    float* sm_m = sm;
    float* sm_l = sm_m + NW * 16;
    float* sm_acc = sm_l + NW * 16;
    const int col = lane % 16;
    const int jgrp = lane / 16;
    if (jgrp == 0) {
        sm_m[wave * 16 + col] = m_run;
        sm_l[wave * 16 + col] = l_tot;
    }
    if (col < group) {
        float* row = sm_acc + (wave * group + col) * kAccStride;
#pragma unroll
        for (int c = 0; c < 8; ++c)
            *reinterpret_cast<f32x4*>(row + 16 * c + 4 * jgrp) = acc_o[c];
    }
    __syncthreads();
    for (int it = wave * 64 + lane; it < group * (kDim / 4); it += NW * 64) {
        const int qh = it / (kDim / 4);
        const int d = (it % (kDim / 4)) * 4;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w * 16 + qh]);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        float lt = 0.f;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = exp2f(sm_m[w * 16 + qh] - M_use);
            lt += f * sm_l[w * 16 + qh];
            o += f * *reinterpret_cast<const f32x4*>(sm_acc + (w * group + qh) * kAccStride + d);
        }
        store(qh, d, M, lt, o);
    }
}

// Combine the partitions of each (request, query head):
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = v_scale * sum_p w_p acc_p / sum_p w_p l_p
// Requests that are aborted, empty, too long, or that a partition marked as
// mapped to an invalid page (l_p < 0) get zeros. A wavefront reduces a row in
// two passes: the first over the (max, sum) pairs finds M and any invalid
// mark; the second takes 64 slots at a time (the next 64 pairs loading
// meanwhile), and a ballot of the nonzero weights lists the slots to read,
// whose outputs (two dims per lane, 512 B per slot) are loaded up to 8 at a
// time before any is accumulated. Empty slots (weight 0) are never read.
// Rows of at most kShortRow slots take a single round trip instead.
constexpr int kReduceWaves = 4;
constexpr int kReduceBatch = 8;             // slot outputs in flight per wavefront (16 requests
                                            // up to 131k tokens: 7.3 us; 4: 8.3, 16: 7.9, 32: 10.9)

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

constexpr f32x2 kEmptySlot = {-INFINITY, 0.f};
// Rows of at most this many slots are combined in one round trip.
constexpr int kShortRow = 16;

// First pass over this wavefront's slots c0 + lane, c0 + lane + cstep, ...
// (< np) of one row's (max, sum) pairs: the lane's maximum and whether any
// slot carries the invalid-page mark. Four loads in flight per lane.
__device__ __forceinline__ void row_slot_max(const f32x2* __restrict__ ml, int np, int c0, int cstep,
                                             int lane, float& mx, bool& bad) {
    mx = -INFINITY;
    bad = false;
    for (int i0 = c0 + lane; i0 < np; i0 += 4 * cstep) {
        f32x2 e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            e[k] = i0 + cstep * k < np ? ml[i0 + cstep * k] : kEmptySlot;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            bad |= e[k][1] < 0.f;
            mx = fmaxf(mx, e[k][0]);
        }
    }
}

// Second pass over the 64-slot chunks c0, c0 + cstep, ... (< np): the lane's
// share of sum_p w_p l_p and its two dims of sum_p w_p acc_p, with
// w_p = 2^(m_p - M_use). acc points at the row's outputs plus 2 * lane.
__device__ __forceinline__ void row_slot_accumulate(const f32x2* __restrict__ ml,
                                                    const float* __restrict__ acc, int np, int c0,
                                                    int cstep, int lane, float M_use, float& lsum,
                                                    f32x2& num) {
    lsum = 0.f;
    num = f32x2{0.f, 0.f};
    f32x2 e_next = c0 + lane < np ? ml[c0 + lane] : kEmptySlot;
    for (int c = c0; c < np; c += cstep) {
        const f32x2 e = e_next;                               // the next chunk's pairs load
        e_next = c + cstep + lane < np ? ml[c + cstep + lane]
                                       : kEmptySlot;          // under this one's reads
        const float w = exp2f(e[0] - M_use);                  // 0 for an empty slot
        lsum += w * e[1];
        uint64_t mask = __builtin_amdgcn_ballot_w64(w > 0.f);
        while (mask != 0) {
            int sl[kReduceBatch];
            f32x2 v[kReduceBatch];
#pragma unroll
            for (int k = 0; k < kReduceBatch; ++k) {
                sl[k] = mask != 0 ? __builtin_ctzll(mask) : -1;    // wave-uniform
                mask &= mask - 1;
                if (sl[k] >= 0)
                    v[k] = *reinterpret_cast<const f32x2*>(
                        acc + static_cast<size_t>(c + sl[k]) * kDim);
            }
#pragma unroll
            for (int k = 0; k < kReduceBatch; ++k) {
                if (sl[k] >= 0)
                    num += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), sl[k])) * v[k];
            }
        }
    }
}

// One wavefront reduces one whole row (slots [0, np)) and writes its two
// dims per lane of the output o (already offset by the lane).
__device__ __forceinline__ void reduce_row_wave(const f32x2* __restrict__ ml,
                                                const float* __restrict__ acc, int np, float vs,
                                                f32x2* o, int lane) {
    if (np <= kShortRow) {
        // one round trip: every (max, sum) pair and every slot's two dims
        // are requested before any is used
        const f32x2 e = lane < np ? ml[lane] : kEmptySlot;
        f32x2 v[kShortRow];
#pragma unroll
        for (int k = 0; k < kShortRow; ++k)              // slots past np re-read the last one
            v[k] = *reinterpret_cast<const f32x2*>(
                acc + static_cast<size_t>(min(k, np - 1)) * kDim);
        if (__builtin_amdgcn_ballot_w64(e[1] < 0.f) != 0) {  // an invalid-page mark
            *o = f32x2{0.f, 0.f};
            return;
        }
        const float M = wave_max(e[0]);
        const float w = exp2f(e[0] - (M == -INFINITY ? 0.f : M));   // 0 for empty slots
        const float lt = wave_sum(w * e[1]);
        f32x2 num = {0.f, 0.f};
#pragma unroll
        for (int k = 0; k < kShortRow; ++k) {
            const f32x2 t = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k)) * v[k];
            num += k < np ? t : f32x2{0.f, 0.f};
        }
        *o = lt > 0.f ? num * (vs / lt) : f32x2{0.f, 0.f};
        return;
    }
    float mx;
    bool bad;
    row_slot_max(ml, np, 0, 64, lane, mx, bad);
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {              // uniform per row
        *o = f32x2{0.f, 0.f};
        return;
    }
    const float M = wave_max(mx);
    float lsum;
    f32x2 num;
    row_slot_accumulate(ml, acc, np, 0, 64, lane, M == -INFINITY ? 0.f : M, lsum, num);
    const float lt = wave_sum(lsum);
    *o = lt > 0.f ? num * (vs / lt) : f32x2{0.f, 0.f};
}

// Shared-mode partition kernel. Grid: blockIdx.x = (p * batch + b) * hkv + g;
// the NW wavefronts of the workgroup share partition p of (b, g) (pairs w,
// w + NW, ...) and merge in LDS. NW = 4, or 8 when the grid has at most one
// workgroup per CU (e.g. 32 requests x 8 KV heads), so each CU still streams
// with 8 wavefronts and no split-K reduction is needed.
// With several partitions each workgroup writes its partial (m, l, acc) and
// reduce_partials_kernel, launched next, combines them. (Combining them in
// the last workgroup of each (b, g) of the same launch, behind device-scope
// stores and a counter, measured 1-3% slower at 1 to 16 requests.)
// Occupancy is pinned at 2 waves per SIMD: the register pipeline needs ~200
// VGPRs, and without the cap the scheduler may trade the in-flight loads for a
// third wave (sinking the prefetches next to their uses), which halves the
// streaming rate. SPLIT: more than one partition (partials written); the
// one-partition instance writes the output and carries no partial code.
template <bool FP8, int NW, bool APPEND, bool SPLIT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_partition_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, uint8_t* __restrict__ k_pool,
    uint8_t* __restrict__ v_pool, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table, int32_t bt_stride,
    const int32_t* __restrict__ seq_lens, int32_t max_seq_len, const uint8_t* __restrict__ abort,
    float* __restrict__ out, float* __restrict__ part_ml, float* __restrict__ part_acc,
    float sm_scale_log2, int32_t batch, int32_t hq, int32_t hkv, int32_t num_pages,
    int32_t part_tokens, int32_t n_parts) {
    extern __shared__ float smem[];
    constexpr int kThreads = NW * 64;
    const int group = hq / hkv;
    // LDS: the merge area, then the page ids of the partition
    int32_t* sm_ids = reinterpret_cast<int32_t*>(smem + merge_floats(NW, group));

    const int bid = blockIdx.x;
    const int g = bid % hkv;
    const int b = (bid / hkv) % batch;
    const int p = bid / (hkv * batch);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // uniform per wavefront
    const int lane = tid % 64;
    const int col = lane % 16;       // query column of the MFMA tiles
    const int jgrp = lane / 16;      // k-group of the operands / row group of the result

    // The loads that do not depend on each other go out together: the
    // request's length, this thread's first page id of the partition (within
    // the table row whatever the length) and the query operand. A short
    // request then waits one memory round trip before its tiles, not three.
    const int t_begin = p * part_tokens;
    const int pg0 = t_begin / kPage;
    const int32_t* bt_row = block_table + static_cast<size_t>(b) * bt_stride + pg0;
    const size_t q_row = static_cast<size_t>(b) * hq + g * group;
    const int L = seq_lens[b];
    int32_t id0 = -1;
    if (tid < part_tokens / kPage && pg0 + tid < bt_stride) id0 = bt_row[tid];
    bf16x8 qop[4];
    load_q_operand(qop, q, q_row, group, col, jgrp);
    const bool ok = request_ok(seq_lens, abort, b, L, max_seq_len, bt_stride);
    if (!ok || static_cast<int64_t>(p) * part_tokens >= L) {
        // A refused request's zeros come from its first partition's
        // workgroup; partitions past a valid request's end have nothing to do.
        if (!ok && p == 0) {
            for (int i = tid; i < group * kDim; i += kThreads)
                out[(static_cast<size_t>(b) * hq + g * group) * kDim + i] = 0.f;
        }
        return;
    }
    const int t_end = min(L, t_begin + part_tokens);
    const int npg = (t_end + kPage - 1) / kPage - pg0;

    // Page ids -> LDS; any id outside the pool poisons the partition (its
    // output, and the request's, becomes zero and none of its pages is read).
    int bad = 0;
    if (tid < npg) {
        bad |= (id0 < 0 || id0 >= num_pages);
        sm_ids[tid] = id0;
    }
    for (int k = tid + kThreads; k < npg; k += kThreads) {
        const int32_t id = bt_row[k];
        bad |= (id < 0 || id >= num_pages);
        sm_ids[k] = id;
    }
    bad = __syncthreads_or(bad);

    float m_run = -INFINITY;
    float l_run = 0.f;
    f32x4 acc_o[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc_o[c] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (!bad) {
        const float s_scale = FP8 ? sm_scale_log2 * k_scale[g] : sm_scale_log2;
        const auto tile_of = [&](int page_idx) __attribute__((always_inline)) -> size_t {
            const int id = __builtin_amdgcn_readfirstlane(sm_ids[page_idx]);
            return static_cast<size_t>(id) * hkv + g;
        };
        const size_t new_row = (static_cast<size_t>(b) * hkv + g) * kDim;
        stream_share<FP8, APPEND, kSharedDepth, NW == 4>(
            tile_of, k_pool, v_pool, npg, pg0, wave, NW, t_begin, t_end, L, lane, jgrp, s_scale,
            qop, k_new + new_row, v_new + new_row, k_scale + g, v_scale + g, m_run, l_run, acc_o);
    }

    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);

    // ---- merge the NW wavefronts -----------------------------------------
    const float vs = (FP8 && v_scale != nullptr) ? v_scale[g] : 1.0f;
    merge_waves<NW>(smem, wave, lane, group, m_run, l_tot, acc_o,
                    [&](int qh, int d, float M, float lt, const f32x4& o) {
        if constexpr (!SPLIT) {
            f32x4 r = {0.f, 0.f, 0.f, 0.f};
            if (!bad && lt > 0.f) r = o * (vs / lt);
            *reinterpret_cast<f32x4*>(out + (q_row + qh) * kDim + d) = r;
        } else {
            const size_t pslot = (q_row + qh) * partial_slots(n_parts) + p;
            *reinterpret_cast<f32x4*>(part_acc + pslot * kDim + d) = o;
            if (d == 0) *reinterpret_cast<f32x2*>(part_ml + 2 * pslot) = f32x2{M, bad ? -1.f : lt};
        }
    });
}

// Persistent kernel for short partitions (<= 2048 tokens), used when there
// are enough of them to give every CU work. The (request, KV head, page)
// units of the requests that have work are numbered request by request, then
// KV head, then page, each (request, KV head) led by kPiecePenalty units that
// hold no page (the cost of one more piece); each workgroup first builds the
// per-request prefix of unit counts in LDS, then workgroup j of the G that
// share the work takes the contiguous range of units [j U / G, (j + 1) U / G),
// so the split is even to within a unit. G is the grid size, lowered if needed so that every range
// holds at least one partition's worth of pages. A range is streamed as runs,
// one per (request, KV head) it touches, cut into pieces of at most
// kCoopRunPages pages that end on partition boundaries. The four wavefronts
// share each piece as in the shared kernel (page pairs w, w + 4, ...), merge
// through LDS and write one partial.
//
// Where the partials go: a piece owns the slot of every partition whose first
// page it streams, and the piece that reaches the end of a (request, KV head)
// also owns the extra slot after its last partition, so every slot of a
// request is owned by exactly one piece. A piece writes its partial to the
// first slot it owns and marks the others empty (max -inf, sum 0), which the
// reduction weighs 0. Only a workgroup's first piece can start inside a
// partition. A range holds at least one partition's worth of units, and the
// units after a page of a (request, KV head) up to its end are all pages, so
// such a piece either reaches the next partition's first page (a piece runs
// to at least the second partition boundary after its start) or ends the
// (request, KV head) inside its last partition and takes the extra slot.
// Aborted, empty or unmappable requests have no units (the reduction writes
// their zeros).
constexpr int kWaveModeMaxBatch = 4096;     // LDS: 2 * batch + 1 ints
constexpr int kCoopRunPages = 1024;         // pages of one piece (LDS page ids)
#ifndef KVFP8_PIECE_PENALTY
#define KVFP8_PIECE_PENALTY 64
#endif
// Units counted at the start of every (request, KV head) on top of its pages:
// the cost of starting a piece (page ids, pipeline fill and drain, LDS merge,
// partial store) in page-equivalents, so shares that cross many short requests
// get fewer pages. Measured on 16 requests of 512 to 131,072 tokens: 8, 12,
// 24, 48, 64, 96 units gave 0.203, 0.197-0.202, 0.195, 0.192, 0.190 and
// 0.190 ms per one-layer step.
constexpr int kPiecePenalty = KVFP8_PIECE_PENALTY;
static_assert(kCoopRunPages >= 2 * (kWaveModeMaxTokens / kPage) - 1,
              "a piece starting inside a partition must reach the next partition's start");

// Dynamic LDS of the persistent kernel: the merge area, the piece's page ids,
// then the per-request prefix and lengths.
__host__ __device__ constexpr size_t coop_lds_bytes(int group, int batch) {
    return sizeof(float) * merge_floats(kWaves, group) +
           sizeof(int32_t) * (kCoopRunPages + 2 * static_cast<size_t>(batch) + 1);
}

template <bool FP8, bool APPEND>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_wave_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, uint8_t* __restrict__ k_pool,
    uint8_t* __restrict__ v_pool, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table, int32_t bt_stride,
    const int32_t* __restrict__ seq_lens, int32_t max_seq_len, const uint8_t* __restrict__ abort,
    float* __restrict__ out, float* __restrict__ part_ml, float* __restrict__ part_acc,
    float sm_scale_log2, int32_t batch, int32_t hq,
    int32_t hkv, int32_t num_pages, int32_t part_tokens, int32_t n_parts) {
    constexpr int kThreads = kWaves * 64;
    extern __shared__ float smem[];
    const int group = hq / hkv;
    int32_t* sm_ids = reinterpret_cast<int32_t*>(smem + merge_floats(kWaves, group));
    int32_t* sm_pre = sm_ids + kCoopRunPages;   // [batch + 1] pages before request b
    int32_t* sm_len = sm_pre + batch + 1;       // [batch] seq_lens
    __shared__ int32_t sm_wsum[kWaves];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64;
    const int col = lane % 16;
    const int jgrp = lane / 16;
    const int ppp = part_tokens / kPage;    // pages per partition
    const int64_t n_slots = partial_slots(n_parts);

    // ---- per-request page counts and their exclusive prefix --------------
    {
        const int per = (batch + kThreads - 1) / kThreads;     // contiguous requests per thread
        const int b0 = tid * per;
        int local = 0;
        for (int k = 0; k < per; ++k) {
            const int b = b0 + k;
            if (b >= batch) break;
            const int L = seq_lens[b];
            sm_len[b] = L;
            if (request_ok(seq_lens, abort, b, L, max_seq_len, bt_stride))
                local += (L + kPage - 1) / kPage + kPiecePenalty;
        }
        int incl = local;                                      // inclusive scan in the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o);
            if (lane >= o) incl += v;
        }
        if (lane == 63) sm_wsum[wave] = incl;
        __syncthreads();
        int before = 0;
        for (int w = 0; w < wave; ++w) before += sm_wsum[w];
        int run = before + incl - local;                       // exclusive prefix of b0
        for (int k = 0; k < per; ++k) {
            const int b = b0 + k;
            if (b >= batch) break;
            sm_pre[b] = run;
            const int L = sm_len[b];
            if (request_ok(seq_lens, abort, b, L, max_seq_len, bt_stride))
                run += (L + kPage - 1) / kPage + kPiecePenalty;
        }
        if (tid == kThreads - 1) {
            int total = 0;
            for (int w = 0; w < kWaves; ++w) total += sm_wsum[w];
            sm_pre[batch] = total;
        }
        __syncthreads();
    }
    // units in request, KV head, page order; workgroup j takes [j U / G, (j + 1) U / G)
    const int64_t n_units = static_cast<int64_t>(sm_pre[batch]) * hkv;
    const int64_t n_groups = min(static_cast<int64_t>(gridDim.x), max<int64_t>(1, n_units / ppp));
    const int64_t blk = blockIdx.x;
    if (blk >= n_groups) return;                               // the whole workgroup
    const int64_t u_end = n_units * (blk + 1) / n_groups;

    for (int64_t it = n_units * blk / n_groups; it < u_end;) {
        int lo = 0, hi = batch - 1;                            // last b with pre[b] * hkv <= it
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if (static_cast<int64_t>(sm_pre[mid]) * hkv <= it) lo = mid;
            else hi = mid - 1;
        }
        const int b = __builtin_amdgcn_readfirstlane(lo);
        const int L = __builtin_amdgcn_readfirstlane(sm_len[b]);
        const int npg_b = (L + kPage - 1) / kPage;
        const int ext_b = npg_b + kPiecePenalty;               // units of one (b, g)
        const int local = static_cast<int>(it - static_cast<int64_t>(sm_pre[b]) * hkv);
        const int g = __builtin_amdgcn_readfirstlane(local / ext_b);
        const int r = __builtin_amdgcn_readfirstlane(local % ext_b);
        if (r < kPiecePenalty) {                               // the (b, g)'s leading units
            it += min(static_cast<int64_t>(kPiecePenalty - r), u_end - it);
            continue;                                          // uniform over the workgroup
        }
        const int k0 = r - kPiecePenalty;
        // the piece: pages k0 .. k_end - 1 of (b, g)
        const int cap = (k0 + kCoopRunPages) / ppp * ppp;
        const int k_end = static_cast<int>(
            min(min(static_cast<int64_t>(npg_b), static_cast<int64_t>(cap)), k0 + (u_end - it)));
        const int npg = k_end - k0;                            // 1 .. kCoopRunPages
        it += npg;
        const int t_begin = k0 * kPage;
        const int t_end = min(L, k_end * kPage);

        // page ids -> LDS; an id outside the pool poisons the request
        int bad = 0;
        {
            const int32_t* bt_row = block_table + static_cast<size_t>(b) * bt_stride + k0;
            for (int k = tid; k < npg; k += kThreads) {
                const int32_t id = bt_row[k];
                bad |= (id < 0 || id >= num_pages);
                sm_ids[k] = id;
            }
        }
        bad = __syncthreads_or(bad);

        const size_t q_row = static_cast<size_t>(b) * hq + g * group;
        float m_run = -INFINITY;
        float l_run = 0.f;
        f32x4 acc_o[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc_o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!bad) {
            bf16x8 qop[4];
            load_q_operand(qop, q, q_row, group, col, jgrp);
            const float s_scale = FP8 ? sm_scale_log2 * k_scale[g] : sm_scale_log2;
            const auto tile_of = [&](int page_idx) __attribute__((always_inline)) -> size_t {
                const int id = __builtin_amdgcn_readfirstlane(sm_ids[page_idx]);
                return static_cast<size_t>(id) * hkv + g;
            };
            const size_t new_row = (static_cast<size_t>(b) * hkv + g) * kDim;
            stream_share<FP8, APPEND, 3, true>(tile_of, k_pool, v_pool, npg, k0, wave, kWaves,
                                                t_begin, t_end, L, lane, jgrp, s_scale, qop,
                                                k_new + new_row, v_new + new_row, k_scale + g,
                                                v_scale + g, m_run, l_run, acc_o);
        }
        float l_tot = l_run + __shfl_xor(l_run, 16);
        l_tot += __shfl_xor(l_tot, 32);
        // owned slots: partitions first_own .. end_own - 1 (their first page is in
        // [k0, k_end)), and the extra slot np_b when the piece ends the (b, g)
        const int first_own = (k0 + ppp - 1) / ppp;
        const int end_own = (k_end + ppp - 1) / ppp;
        const int np_b = (npg_b + ppp - 1) / ppp;
        const bool owns_extra = k_end == npg_b;
        const int dst = first_own < end_own ? first_own : np_b;
        merge_waves<kWaves>(smem, wave, lane, group, m_run, l_tot, acc_o,
                            [&](int qh, int d, float M, float lt, const f32x4& o) {
            const size_t row = (q_row + qh) * n_slots;
            *reinterpret_cast<f32x4*>(part_acc + (row + dst) * kDim + d) = o;
            if (d == 0) {
                part_ml[2 * (row + dst)] = M;
                part_ml[2 * (row + dst) + 1] = bad ? -1.f : lt;
                for (int s = first_own; s < end_own; ++s) {
                    if (s == dst) continue;
                    part_ml[2 * (row + s)] = -INFINITY;
                    part_ml[2 * (row + s) + 1] = 0.f;
                }
                if (owns_extra && dst != np_b) {
                    part_ml[2 * (row + np_b)] = -INFINITY;
                    part_ml[2 * (row + np_b) + 1] = 0.f;
                }
            }
        });
        __syncthreads();            // the next piece rewrites the ids and the merge area
    }
}

// COOP = false: one wavefront per (b, h), four rows per workgroup. COOP = true
// (rows of more than 64 slots): one row per workgroup, its four wavefronts
// taking every fourth 64-slot chunk; they agree on M (and any invalid mark)
// through LDS, then wavefront 0 adds the four partial sums.
template <bool COOP>
__global__ __launch_bounds__(kReduceWaves * 64) void reduce_partials_kernel(
    const float* __restrict__ part_ml, const float* __restrict__ part_acc,
    const int32_t* __restrict__ seq_lens, int32_t max_seq_len, int32_t bt_stride,
    const uint8_t* __restrict__ abort, const float* __restrict__ v_scale,
    float* __restrict__ out, int32_t batch, int32_t hq, int32_t hkv, int32_t part_tokens,
    int32_t n_parts, int32_t extra_slot) {
    __shared__ float sm_max[kReduceWaves];
    __shared__ int sm_bad[kReduceWaves];
    __shared__ float sm_sum[kReduceWaves];
    __shared__ f32x2 sm_num[COOP ? kReduceWaves : 1][64];
    const int lane = threadIdx.x % 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int64_t bh = COOP ? static_cast<int64_t>(blockIdx.x)
                            : static_cast<int64_t>(blockIdx.x) * kReduceWaves + wave;
    if (bh >= static_cast<int64_t>(batch) * hq) return;       // uniform per row
    const int b = static_cast<int>(bh / hq);
    const int h = static_cast<int>(bh % hq);
    f32x2* o = reinterpret_cast<f32x2*>(out + bh * kDim) + lane;
    const int L = seq_lens[b];
    const bool aborted = abort != nullptr && abort[b] != 0;
    if (aborted || L < 1 || L > max_seq_len ||
        (static_cast<int64_t>(L) + kPage - 1) / kPage > bt_stride) {
        if (!COOP || wave == 0) *o = f32x2{0.f, 0.f};
        return;
    }
    // the request's partitions, plus the slot after them when the persistent
    // kernel may have written it
    const int np = (L + part_tokens - 1) / part_tokens + extra_slot;
    const size_t n_slots = partial_slots(n_parts);
    const f32x2* ml = reinterpret_cast<const f32x2*>(part_ml) + bh * n_slots;
    const float* acc = part_acc + bh * n_slots * kDim + 2 * lane;
    const float vs = v_scale != nullptr ? v_scale[h / (hq / hkv)] : 1.0f;
    if constexpr (!COOP) {
        reduce_row_wave(ml, acc, np, vs, o, lane);
    } else {
        // this wavefront's 64-slot chunks: 64 wave, 64 wave + 256, ...
        constexpr int cstep = 64 * kReduceWaves;
        float mx;
        bool bad;
        row_slot_max(ml, np, 64 * wave, cstep, lane, mx, bad);
        const bool wave_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
        float M = wave_max(mx);
        if (lane == 0) {
            sm_max[wave] = M;
            sm_bad[wave] = wave_bad;
        }
        __syncthreads();
        bool any_bad = false;
        for (int w = 0; w < kReduceWaves; ++w) {
            M = fmaxf(M, sm_max[w]);
            any_bad |= sm_bad[w] != 0;
        }
        if (any_bad) {                                        // uniform per row
            if (wave == 0) *o = f32x2{0.f, 0.f};
            return;
        }
        float lsum;
        f32x2 num;
        row_slot_accumulate(ml, acc, np, 64 * wave, cstep, lane, M == -INFINITY ? 0.f : M, lsum,
                            num);
        sm_num[wave][lane] = num;
        const float ls = wave_sum(lsum);
        if (lane == 0) sm_sum[wave] = ls;
        __syncthreads();
        if (wave != 0) return;
        float lt = 0.f;
        num = f32x2{0.f, 0.f};
        for (int w = 0; w < kReduceWaves; ++w) {
            lt += sm_sum[w];
            num += sm_num[w][lane];
        }
        *o = lt > 0.f ? num * (vs / lt) : f32x2{0.f, 0.f};
    }
}

// gfx950 (MI355X) has 256 CUs; a grid of at most this many workgroups runs
// one per CU.
constexpr int64_t kNumCUs = 256;
// LDS one workgroup may allocate without opting in to more.
constexpr size_t kMaxLdsBytes = 64 * 1024;

// The persistent kernel (even split of the pages over the workgroups) runs
// when there is more than one partition and enough of them for at least one
// 4-wave workgroup per CU, and its LDS (merge area, page ids, two ints per
// request) fits a workgroup.
bool use_wave_partitions(const AttnArgs& a) {
    const int64_t items = static_cast<int64_t>(a.batch) * a.num_kv_heads;
    return a.num_partitions > 1 && a.partition_tokens <= kWaveModeMaxTokens &&
           a.batch <= kWaveModeMaxBatch && items * a.num_partitions >= kWaves * kNumCUs &&
           coop_lds_bytes(a.num_q_heads / a.num_kv_heads, a.batch) <= kMaxLdsBytes;
}

// Shared mode with 8 wavefronts when the grid has at most one workgroup per
// CU. Limited to GQA groups of up to 8 query heads, which keeps the merge's
// LDS (8 waves x group x 132 floats) within the default 64 KiB per workgroup.
bool use_wide_workgroups(const AttnArgs& a) {
    const int64_t items = static_cast<int64_t>(a.batch) * a.num_kv_heads;
    return !use_wave_partitions(a) && items * a.num_partitions <= kNumCUs &&
           a.num_q_heads / a.num_kv_heads <= 8;
}

hipError_t launch_decode_attn(bool fp8, const AttnArgs& a, hipStream_t stream) {
    const int group = a.num_q_heads / a.num_kv_heads;
    const float sm_log2 = a.sm_scale * kLog2e;
    const bool append = a.k_new != nullptr;
    const int64_t items = static_cast<int64_t>(a.batch) * a.num_kv_heads;
#define KVFP8_ARGS                                                                               \
    a.q, a.k_new, a.v_new, static_cast<uint8_t*>(a.k_pool), static_cast<uint8_t*>(a.v_pool),    \
        fp8 ? a.k_scale : nullptr, fp8 ? a.v_scale : nullptr, a.block_table, a.bt_stride,        \
        a.seq_lens, a.max_seq_len, a.abort, a.out, a.part_ml, a.part_acc, sm_log2,              \
        a.batch, a.num_q_heads, a.num_kv_heads, a.num_pages, a.partition_tokens, a.num_partitions
    if (use_wave_partitions(a)) {
        // persistent: at most 2 workgroups per CU, each streams its range of pages
        const int64_t wgs = std::min<int64_t>(2 * kNumCUs,
                                              (items * a.num_partitions + kWaves - 1) / kWaves);
        const size_t lds = coop_lds_bytes(group, a.batch);
#define KVFP8_WAVE(F8, AP)                                                                       \
    hipLaunchKernelGGL((attn_wave_kernel<F8, AP>), dim3(static_cast<uint32_t>(wgs)),            \
                       dim3(kWaves * 64), lds, stream, KVFP8_ARGS)
        if (fp8) {
            if (append) KVFP8_WAVE(true, true); else KVFP8_WAVE(true, false);
        } else {
            if (append) KVFP8_WAVE(false, true); else KVFP8_WAVE(false, false);
        }
#undef KVFP8_WAVE
    } else {
        const int nw = use_wide_workgroups(a) ? kWavesWide : kWaves;
        const size_t lds = sizeof(float) * merge_floats(nw, group) +
                           sizeof(int32_t) * static_cast<size_t>(a.partition_tokens / kPage);
        const dim3 grid(static_cast<uint32_t>(a.num_partitions * items));
        const bool split = a.num_partitions > 1;
#define KVFP8_SHARED(F8, NW, AP, MD)                                                             \
    hipLaunchKernelGGL((attn_partition_kernel<F8, NW, AP, MD>), grid, dim3(NW * 64), lds,       \
                       stream, KVFP8_ARGS)
#define KVFP8_SHARED1(F8, NW, AP)                                 \
    do {                                                          \
        if (split) KVFP8_SHARED(F8, NW, AP, true);                \
        else KVFP8_SHARED(F8, NW, AP, false);                     \
    } while (0)
#define KVFP8_SHARED2(F8, NW)                                     \
    do {                                                          \
        if (append) KVFP8_SHARED1(F8, NW, true);                  \
        else KVFP8_SHARED1(F8, NW, false);                        \
    } while (0)
        if (fp8) {
            if (nw == kWavesWide) KVFP8_SHARED2(true, kWavesWide); else KVFP8_SHARED2(true, kWaves);
        } else {
            if (nw == kWavesWide) KVFP8_SHARED2(false, kWavesWide); else KVFP8_SHARED2(false, kWaves);
        }
#undef KVFP8_SHARED2
#undef KVFP8_SHARED1
#undef KVFP8_SHARED
    }
#undef KVFP8_ARGS
    hipError_t e = hipGetLastError();
    // with several partitions, either kernel leaves its partials to the reduction
    const bool wave = use_wave_partitions(a);
    if (e != hipSuccess || a.num_partitions == 1) return e;
    const int64_t rows = static_cast<int64_t>(a.batch) * a.num_q_heads;
    const int extra = wave ? 1 : 0;  // the persistent kernel's slot after the last partition
#define KVFP8_REDUCE(CO, WGS)                                                                    \
    hipLaunchKernelGGL(reduce_partials_kernel<CO>, dim3(static_cast<uint32_t>(WGS)),             \
                       dim3(kReduceWaves * 64), 0, stream, a.part_ml, a.part_acc, a.seq_lens,    \
                       a.max_seq_len, a.bt_stride, a.abort, fp8 ? a.v_scale : nullptr, a.out,    \
                       a.batch, a.num_q_heads, a.num_kv_heads, a.partition_tokens,               \
                       a.num_partitions, extra)
    if (a.num_partitions + extra > 64) KVFP8_REDUCE(true, rows);
    else KVFP8_REDUCE(false, (rows + kReduceWaves - 1) / kReduceWaves);
#undef KVFP8_REDUCE
    return hipGetLastError();
}

}  // namespace kvfp8
