"""Pins for the oracle's E4M3 codec (CPU only).

The pages name the format only ("FP8 e4m3"); the largest finite value 448 and
the OCP E4M3 bit layout fix the rest. Each test below pins the oracle to
something outside itself: the OCP specification's stated values, torch's own
float8_e4m3fn type, exact rational arithmetic, or a second encoder written at
the bit level.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ocp_e4m3_values.txt")

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def all_bf16_values():
    return e4m3.bf16_bits_to_f64(ALL_BF16)


def test_decode_matches_ocp_spot_values():
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 10
    for code_s, val_s in rows:
        code = int(code_s, 16)
        got = e4m3.DECODE[code]
        if val_s == "nan":
            assert math.isnan(got), code_s
        else:
            want = float(val_s)
            assert got == want, (code_s, got, want)
            assert math.copysign(1.0, got) == math.copysign(1.0, want)


def test_decode_table_shape():
    d = e4m3.DECODE
    assert np.isnan(d).sum() == 2 and np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    fin = d[~np.isnan(d)]
    assert fin.size == 254
    mags = d[:0x7F]
    assert np.all(np.diff(mags) > 0), "non-negative codes must increase"
    assert np.array_equal(d[0x80:0xFF], -d[0x00:0x7F])
    # spacing: 8 subnormal steps of 2^-9, then 8 values per binade
    assert np.allclose(np.diff(mags[:9]), 2.0 ** -9)


def test_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.DECODE
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], ours[m])
    assert np.array_equal(np.signbit(ref[m]), np.signbit(ours[m]))


def test_round_trip_every_code():
    codes = np.arange(256)
    back = e4m3.encode(e4m3.DECODE)
    for c in codes:
        if c in (0x7F, 0xFF):
            assert back[c] == c            # NaN keeps its sign bit
        else:
            assert back[c] == c, hex(c)
            assert e4m3.encode_bruteforce(e4m3.DECODE[c]) == c
            assert e4m3.encode_bitlevel(e4m3.DECODE[c]) == c


def _bruteforce_vectorised(y):
    """argmin over all 127 magnitudes, ties to the even code, by full comparison."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    mags = e4m3.DECODE[:0x7F]
    err = np.abs(mags[None, :] - np.where(np.isnan(a), 0, a)[:, None])
    best = err.min(axis=1, keepdims=True)
    cand = err == best
    even_cand = cand & (np.arange(0x7F)[None, :] % 2 == 0)
    pick = np.where(even_cand.any(axis=1), even_cand.argmax(axis=1), cand.argmax(axis=1))
    pick = np.where(a >= 448.0, 0x7E, pick)
    sign = np.where(np.signbit(y), 0x80, 0)
    out = pick | sign
    out = np.where(np.isnan(y), 0x7F | sign, out)
    return out.astype(np.uint8)


@pytest.mark.parametrize("scale", [1.0, 0.5, 2.0 ** -7, 3.0, 0.009709821, 1.7e-3, 7.25])
def test_three_encoders_agree_on_every_bf16(scale):
    y = all_bf16_values() / np.float64(np.float32(scale))
    a = e4m3.encode(y)
    b = e4m3.encode_bitlevel(y)
    c = _bruteforce_vectorised(y)
    assert np.array_equal(a, b)
    assert np.array_equal(a, c)


def test_scalar_bruteforce_on_sample():
    rng = np.random.default_rng(7)
    y = np.concatenate([rng.normal(0, 50, 300), rng.normal(0, 0.01, 300),
                        e4m3.DECODE[:0x7F] + 2.0 ** -12, [0.0, -0.0, 1e-30, -1e-30]])
    want = np.array([e4m3.encode_bruteforce(v) for v in y], dtype=np.uint8)
    assert np.array_equal(e4m3.encode(y), want)


def test_ties_go_to_even_and_are_exercised():
    mags = e4m3.DECODE[:0x7F]
    mids = (mags[:-1] + mags[1:]) / 2.0
    codes = e4m3.encode(mids)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(codes, want)
    # the exhaustive bf16 set at scale 1 contains every midpoint below 448
    ys = set(all_bf16_values().tolist())
    assert all(m in ys for m in mids)


def test_encode_matches_torch_cast_where_torch_saturation_does_not_differ():
    y = all_bf16_values()
    ok = ~np.isnan(y) & (np.abs(y) <= 464.0)
    yt = torch.from_numpy(y[ok].astype(np.float32))
    ref = yt.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.encode(y[ok]), ref)


def test_saturation_and_specials():
    enc = lambda v: int(e4m3.encode(np.array([v]))[0])  # noqa: E731
    assert enc(448.0) == 0x7E and enc(-448.0) == 0xFE
    assert enc(449.0) == 0x7E and enc(464.0) == 0x7E and enc(465.0) == 0x7E
    assert enc(1e30) == 0x7E and enc(-1e30) == 0xFE
    assert enc(np.inf) == 0x7E and enc(-np.inf) == 0xFE
    assert enc(np.nan) == 0x7F and enc(-np.nan) == 0xFF
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80
    assert enc(2.0 ** -11) == 0x00 and enc(-(2.0 ** -11)) == 0x80   # below half the min subnormal
    assert enc(2.0 ** -10) == 0x00                                  # exact tie 0 vs 2^-9 -> even
    assert enc(3 * 2.0 ** -11) == 0x01
    assert enc(1.0625) == 0x38 and enc(1.1875) == 0x3A              # ties to even mantissa
    assert enc(432.0) == 0x7E                                       # tie 416/448 -> even (0x7E)


def test_encode_is_monotone():
    y = np.sort(np.concatenate([np.linspace(-500, 500, 200001), all_bf16_values()]))
    y = y[~np.isnan(y)]
    v = e4m3.DECODE[e4m3.encode(y)]
    assert np.all(np.diff(v) >= 0)


def _rne_exact(q: Fraction) -> int:
    """Code of the exact rational q, by exact comparisons with every code."""
    sign = 0x80 if q < 0 else 0
    a = abs(q)
    if a >= 448:
        return 0x7E | sign
    best = None
    for c in range(0x7F):
        err = abs(Fraction(e4m3.DECODE[c]) - a)
        if best is None or err < best[1] or (err == best[1] and c % 2 == 0):
            best = (c, err)
    return best[0] | sign


def test_quantize_equals_rounding_the_exact_quotient():
    rng = np.random.default_rng(11)
    xs = rng.choice(ALL_BF16, size=400)
    xs = xs[~np.isnan(e4m3.bf16_bits_to_f64(xs))]
    scales = np.concatenate([rng.uniform(1e-3, 2e-2, 10), [1.0, 0.25, 3.0]]).astype(np.float32)
    for s in scales:
        got = e4m3.quantize(xs, s)
        for x_bits, g in zip(xs, got):
            x = e4m3.bf16_bits_to_f64(np.array([x_bits]))[0]
            if math.isinf(x):
                continue
            q = Fraction(x) / Fraction(float(s))
            want = _rne_exact(q)
            if q == 0 and math.copysign(1, x) < 0:
                want = 0x80
            assert g == want, (hex(int(x_bits)), float(s))


def test_planted_tie_rule_mistake_is_caught():
    """A ties-away encoder (a plausible slip) must differ on the bf16 set."""
    y = all_bf16_values()
    a = np.abs(np.where(np.isnan(y), 0, y))
    mags = e4m3.DECODE[:0x7F]
    hi = np.clip(np.searchsorted(mags, a), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    tie_away = np.where(np.abs(mags[lo] - a) < np.abs(mags[hi] - a), lo, hi)
    tie_away = np.where(a >= 448, 0x7E, tie_away).astype(np.uint8)
    good = e4m3.encode(np.abs(y)) & 0x7F
    assert np.any(tie_away[~np.isnan(y)] != good[~np.isnan(y)])


def _amax_scales(n=40, seed=5):
    """fp32(amax / 448) for bf16 amax values: the scale shape the cache uses."""
    rng = np.random.default_rng(seed)
    v = all_bf16_values()
    cand = np.unique(np.abs(v[np.isfinite(v) & (np.abs(v) > 1e-3) & (np.abs(v) < 1e3)]))
    return (rng.choice(cand, size=n, replace=False).astype(np.float32) / np.float32(448))


def test_quantize_is_exact_on_every_near_tie_of_amax_scales():
    """With s = amax/448 the exact quotient often sits a hair off an E4M3
    midpoint. Every such near-tie (float64 quotient within 2^-30 relative of
    a midpoint) is checked against exact rational rounding."""
    x_bits = ALL_BF16[np.isfinite(all_bf16_values())]
    x = e4m3.bf16_bits_to_f64(x_bits)
    mags = e4m3.DECODE[:0x7F]
    mids = (mags[:-1] + mags[1:]) / 2
    checked = 0
    for s in _amax_scales():
        q = np.abs(x / np.float64(s))
        i = np.clip(np.searchsorted(mids, q), 1, len(mids) - 1)
        near = np.minimum(np.abs(q - mids[i - 1]), np.abs(q - mids[i])) <= q * 2.0 ** -30
        got = e4m3.quantize(x_bits[near], s)
        for xb, g in zip(x_bits[near], got):
            xv = e4m3.bf16_bits_to_f64(np.array([xb]))[0]
            assert g == _rne_exact(Fraction(xv) / Fraction(float(s))), (hex(int(xb)), float(s))
            checked += 1
    assert checked > 100


def test_plain_fp32_quotient_would_double_round():
    """The trap the GPU encoder must avoid: rounding the correctly rounded
    fp32 quotient gives wrong codes for amax/448 scales (so a GPU encoder
    that passes the exhaustive test with these scales is not doing that)."""
    x_bits = ALL_BF16[np.isfinite(all_bf16_values())]
    x32 = e4m3.bf16_bits_to_f64(x_bits).astype(np.float32)
    wrong = 0
    with np.errstate(over="ignore"):
        for s in _amax_scales(12):
            plain = e4m3.encode((x32 / np.float32(s)).astype(np.float64))
            wrong += int((plain != e4m3.quantize(x_bits, s)).sum())
    assert wrong > 0
