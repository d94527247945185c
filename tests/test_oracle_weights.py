"""Pins for the weight-quantization oracle (INT4 / FP8 weights) and its GEMV.

Ties it to things outside itself: a pure-Python loop over struct-decoded
values, groups built from exactly representable values (closed forms,
including ties that must go to even), exact rational arithmetic for the
scales, the error bound of round-to-nearest, and a one-hot activation that
reads back one column of the dequantized weights.
"""

import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, weights

G = weights.GROUP


def _bf16(x):
    x = np.asarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)          # exact for bf16-representable x


def _val(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _rand_w(rng, n, k, sigma=0.02):
    x = rng.normal(0, sigma, size=(n, k)).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def test_gemv_matches_python_loop():
    rng = np.random.default_rng(0)
    M, N, K = 2, 3, 256
    wb = _rand_w(rng, N, K)
    xb = _rand_w(rng, M, K, sigma=1.0)
    q, s = weights.quantize_int4(wb)
    y = weights.gemv(xb, weights.dequant_int4(q, s))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += _val(xb[m, k]) * int(q[n, k]) * float(s[n, k // G])
            assert y[m, n] == pytest.approx(acc, rel=1e-12, abs=1e-15)


def test_int4_exactly_representable_groups_and_ties_to_even():
    # one group with amax = 7 * 2^-6: s = 2^-6 exactly; multiples of s come back unchanged
    s0 = 2.0 ** -6
    qs = np.array([7, -7, 0, 3, -3, 1, -1, 5] * (G // 8))
    w = _bf16(qs * s0)[None, :]
    q, s = weights.quantize_int4(w)
    assert s[0, 0] == np.float32(s0) and np.array_equal(q[0], qs)
    # halves go to the even neighbour; amax stays 7 s
    ties = np.array([7.0, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5] * (G // 8))
    q, s = weights.quantize_int4(_bf16(ties * s0)[None, :])
    assert np.array_equal(q[0, :8], [7, 2, 4, -2, -4, 0, 0, 2])
    # an all-zero group: scale 1, codes 0
    q, s = weights.quantize_int4(np.zeros((1, G), np.uint16))
    assert s[0, 0] == 1.0 and not q.any()


def _nearest_fp32(qv: Fraction):
    c = np.float32(float(qv))
    best = None
    for cand in (np.nextafter(c, np.float32(0)), c, np.nextafter(c, np.float32(np.inf))):
        key = (abs(Fraction(float(cand)) - qv), int(cand.view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def test_scales_and_rounding_bounds_on_random_weights():
    rng = np.random.default_rng(1)
    wb = _rand_w(rng, 16, 4 * G)
    q, s = weights.quantize_int4(wb)
    qf, sf = weights.quantize_fp8(wb)
    w = e4m3.bf16_bits_to_f64(wb).reshape(16, 4, G)
    for n in range(16):
        for g in range(4):
            amax = Fraction(float(np.abs(w[n, g]).max()))
            assert s[n, g] == _nearest_fp32(amax / 7)
            assert sf[n, g] == _nearest_fp32(amax / 448)
    assert q.min() >= -8 and q.max() <= 7
    err = np.abs(w - weights.dequant_int4(q, s).reshape(16, 4, G))
    assert np.all(err <= s.astype(np.float64)[:, :, None] / 2 * (1 + 1e-12))
    # FP8 codes are the KV encoder's codes of w / s
    want = e4m3.quantize(wb.reshape(16, 4, G), sf[:, :, None]).reshape(16, 4 * G)
    assert np.array_equal(qf, want)


@pytest.mark.parametrize("fmt", ["int4", "fp8"])
def test_one_hot_activation_reads_a_column(fmt):
    rng = np.random.default_rng(2)
    wb = _rand_w(rng, 5, 2 * G)
    if fmt == "int4":
        q, s = weights.quantize_int4(wb)
        wd = weights.dequant_int4(q, s)
    else:
        q, s = weights.quantize_fp8(wb)
        wd = weights.dequant_fp8(q, s)
    x = np.zeros((1, 2 * G), np.uint16)
    x[0, 200] = 0x3F80                                      # 1.0
    y = weights.gemv(x, wd)
    assert np.array_equal(y[0], wd[:, 200])


def test_int4_codes_never_reach_minus_8():
    """|w / s| <= amax / fp32(amax / 7) < 7.5 for every finite bf16 amax, so
    the INT4 codes stay in [-7, 7] and three magnitude bits and a sign bit
    hold every code (the packed format is sign-magnitude). Exhaustive over the
    amax patterns; then groups whose most negative value is -amax, quantized
    by the oracle."""
    a_bits = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)     # every positive finite
    amax = e4m3.bf16_bits_to_f64(a_bits)
    s = (amax / 7.0).astype(np.float32).astype(np.float64)
    ratio = [Fraction(float(a)) / Fraction(float(t)) for a, t in zip(amax[::97], s[::97])]
    assert max(ratio) < Fraction(15, 2)
    assert np.all(amax / s < 7.5 * (1 - 1e-12))
    rng = np.random.default_rng(7)
    pick = a_bits[rng.choice(a_bits.size, size=4 * 64, replace=False)]
    w = _rand_w(rng, 4 * 64, G)
    w[:, 0] = pick | 0x8000                                     # -amax somewhere in each group
    w[:, 1:] = np.where((w[:, 1:] & 0x7FFF) > pick[:, None], w[:, 1:] & 0x8000, w[:, 1:])
    q, _ = weights.quantize_int4(w)
    assert q.min() == -7 and q.max() <= 7
