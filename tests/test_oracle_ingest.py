"""Pins for the oracle's prefill ingest: amax, scales and the page writer (CPU).

Each test ties the oracle to something outside itself: a bf16 decode through
the struct module and plain Python max, exact rational arithmetic for the
scale quotient, and the token-by-token append oracle (pinned separately)
for the page writer.
"""

import math
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, ingest, paged

P = 16


def _bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _random_bf16(rng, shape, specials=True):
    x = rng.normal(0.0, 2.0, size=shape).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    if specials:
        flat = bits.reshape(-1)
        idx = rng.choice(flat.size, size=max(1, flat.size // 50), replace=False)
        flat[idx] = rng.choice(np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x7F81, 0x8000],
                                        dtype=np.uint16), size=idx.size)
    return bits


# ---------------------------------------------------------------------------
# amax
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(7, 3, 8), (1, 1, 128), (33, 2, 16)])
def test_amax_matches_struct_bruteforce(shape):
    rng = np.random.default_rng(sum(shape))
    bits = _random_bf16(rng, shape)
    got = ingest.amax_finite(bits)
    for g in range(shape[1]):
        best = 0.0
        for r in range(shape[0]):
            for d in range(shape[2]):
                v = _bf16_value(bits[r, g, d])
                if math.isfinite(v):
                    best = max(best, abs(v))
        assert float(got[g]) == best


def test_amax_known_values():
    z = np.zeros((4, 2, 8), np.uint16)
    assert np.array_equal(ingest.amax_finite(z), [0.0, 0.0])
    nan_inf = np.full((4, 2, 8), 0x7FC0, np.uint16)
    nan_inf[:, 1] = 0xFF80                                 # -inf
    assert np.array_equal(ingest.amax_finite(nan_inf), [0.0, 0.0])
    assert ingest.amax_finite(np.zeros((0, 3, 8), np.uint16)).shape == (3,)
    x = np.full((5, 2, 8), 0x3F80, np.uint16)               # 1.0 everywhere
    x[3, 0, 5] = 0xC0A0                                    # -5.0: largest magnitude in head 0
    x[0, 1, 0] = 0x7F7F                                    # largest finite bf16 in head 1
    x[1, 1, 1] = 0x7F80                                    # +inf is skipped
    got = ingest.amax_finite(x)
    assert float(got[0]) == 5.0
    assert float(got[1]) == _bf16_value(0x7F7F) == float(np.float32(3.3895313892515355e38))


# ---------------------------------------------------------------------------
# scales
# ---------------------------------------------------------------------------
def _nearest_fp32_exact(q: Fraction) -> np.float32:
    """The fp32 nearest to the positive rational q, ties to the even
    significand, found by comparing neighbours in exact arithmetic."""
    c = np.float32(float(q))
    best = None
    for cand in (np.nextafter(c, np.float32(0)), c, np.nextafter(c, np.float32(np.inf))):
        err = abs(Fraction(float(cand)) - q)
        key = (err, int(cand.view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def test_scales_are_correctly_rounded_quotients():
    rng = np.random.default_rng(7)
    # bf16 magnitudes (what amax produces) and arbitrary fp32 values
    a16 = (rng.integers(0x0080, 0x7F80, size=400).astype(np.uint32) << 16).view(np.float32)
    a32 = rng.integers(0x00800000, 0x7F800000, size=400).astype(np.uint32).view(np.float32)
    for a in np.concatenate([a16, a32]):
        s = ingest.scales_from_amax(np.array([a]))[0]
        want = _nearest_fp32_exact(Fraction(float(a)) / 448)
        want = max(want, ingest.FLT_MIN)
        assert s.view(np.uint32) == np.float32(want).view(np.uint32), a


def test_scale_special_cases():
    f = lambda v: float(ingest.scales_from_amax(np.array([v], np.float32))[0])
    assert f(0.0) == 1.0
    assert f(np.nan) == 1.0 and f(np.inf) == 1.0 and f(-3.0) == 1.0
    assert f(448.0) == 1.0 and f(224.0) == 0.5 and f(896.0) == 2.0
    assert f(_bf16_value(0x0001)) == float(ingest.FLT_MIN)          # tiny amax: raised
    assert f(448.0 * 2.0 ** -126) == float(ingest.FLT_MIN)
    big = f(_bf16_value(0x7F7F))
    assert math.isfinite(big) and big > 0


# ---------------------------------------------------------------------------
# page writer
# ---------------------------------------------------------------------------
def _ingest_case(rng, cache, lens, hkv=2, d=8, pool_pages=24, stride_extra=1):
    need = [max(1, -(-L // P)) for L in lens]
    perm = rng.permutation(pool_pages).astype(np.int32)
    bt = np.full((len(lens), max(need) + stride_extra), -1, np.int32)
    off = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[off:off + n]
        off += n
    if cache == "fp8":
        kp = rng.integers(0, 256, (pool_pages, hkv, P, d)).astype(np.uint8)
    else:
        kp = rng.integers(0, 65536, (pool_pages, hkv, P, d)).astype(np.uint16)
    vp = kp[::-1].copy()
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64) + 3   # rows 0..2 unused
    rows = int(starts[-1] + lens[-1]) + 2
    k_rows = _random_bf16(rng, (rows, hkv, d), specials=False)
    v_rows = _random_bf16(rng, (rows, hkv, d), specials=False)
    ks = ingest.scales_from_amax(ingest.amax_finite(k_rows))
    vs = ingest.scales_from_amax(ingest.amax_finite(v_rows))
    return bt, kp, vp, starts, k_rows, v_rows, ks, vs


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_ingest_equals_tokenwise_append_with_zero_tails(cache):
    rng = np.random.default_rng(11)
    lens = [37, 0, 16, 1, 17, 33]
    bt, kp, vp, starts, kr, vr, ks, vs = _ingest_case(rng, cache, lens)
    got_k, got_v = kp.copy(), vp.copy()
    ingest.ingest(got_k, got_v, kr, vr, starts, np.array(lens), bt, cache, ks, vs)
    # the same through the token-by-token append oracle, then the zero tails
    want_k, want_v = kp.copy(), vp.copy()
    seq = np.concatenate([np.full(L, b) for b, L in enumerate(lens)])
    pos = np.concatenate([np.arange(L) for L in lens])
    rows = np.concatenate([starts[b] + np.arange(L) for b, L in enumerate(lens)]).astype(np.int64)
    if cache == "fp8":
        paged.append_fp8(want_k, want_v, kr[rows], vr[rows], seq, pos, bt, ks, vs)
    else:
        paged.append_bf16(want_k, want_v, kr[rows], vr[rows], seq, pos, bt)
    for b, L in enumerate(lens):
        if L > 0 and L % P:
            page = bt[b, (L - 1) // P]
            want_k[page, :, L % P:, :] = 0
            want_v[page, :, L % P:, :] = 0
    assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v)
    # pages of no request (and request 1, which is empty) are untouched
    used = {int(bt[b, j]) for b, L in enumerate(lens) for j in range(-(-L // P))}
    for p in set(range(kp.shape[0])) - used:
        assert np.array_equal(got_k[p], kp[p]) and np.array_equal(got_v[p], vp[p])


def test_ingest_skips_aborted_bad_pages_and_overlong():
    rng = np.random.default_rng(12)
    lens = [40, 20, 9]
    bt, kp, vp, starts, kr, vr, ks, vs = _ingest_case(rng, "fp8", lens, stride_extra=0)
    bad_page = int(bt[0, 1])
    bt[0, 1] = 10 ** 6                                   # request 0: its second page is bad
    abort = np.array([0, 1, 0], np.uint8)                # request 1 aborted
    got_k, got_v = kp.copy(), vp.copy()
    ingest.ingest(got_k, got_v, kr, vr, starts, np.array([40, 20, 3 * P + 1]), bt, "fp8",
                  ks, vs, abort=abort)
    # request 0: pages 0 and 2 written, the bad one skipped (its old page untouched)
    for j in (0, 2):
        assert not np.array_equal(got_k[bt[0, j]], kp[bt[0, j]])
    assert np.array_equal(got_k[bad_page], kp[bad_page])
    # a length limit refuses the longer requests whole
    lim_k, lim_v = kp.copy(), vp.copy()
    ingest.ingest(lim_k, lim_v, kr, vr, starts, np.array([40, 20, 9]), bt, "fp8", ks, vs,
                  max_seq_len=20)
    assert np.array_equal(lim_k[bt[0, 0]], kp[bt[0, 0]])             # 40 > 20: untouched
    assert not np.array_equal(lim_k[bt[1, 0]], kp[bt[1, 0]])         # 20 <= 20: written
    # rows past the end of the inputs refuse the request whole
    oob_k, oob_v = kp.copy(), vp.copy()
    starts2 = starts.copy()
    starts2[1] = kr.shape[0] - 19                              # needs 20 rows
    ingest.ingest(oob_k, oob_v, kr, vr, starts2, np.array([40, 20, 9]), bt, "fp8", ks, vs)
    assert np.array_equal(oob_k[bt[1, 0]], kp[bt[1, 0]])
    assert not np.array_equal(oob_k[bt[2, 0]], kp[bt[2, 0]])
    # request 1 (aborted) and request 2 (needs 4 pages, its row holds 3) untouched
    for b in (1, 2):
        for j in range(bt.shape[1]):
            p = int(bt[b, j])
            if 0 <= p < kp.shape[0]:
                assert np.array_equal(got_k[p], kp[p]) and np.array_equal(got_v[p], vp[p])
