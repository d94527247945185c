"""OCP FP8 E4M3 ("e4m3fn") codec, written from the format definition.

TEST INFRASTRUCTURE (see the package docstring): never used by the product path.

Which format: the pages name only FP8 e4m3 as the cache's storage format, in
place of BF16 (remio.ai/it, "Il serving di modelli più piccoli di Cloudflare riduce
la memoria, ma la sicurezza diventa la prova decisiva", section "Cosa ha
cambiato Cloudflare per Kimi e GLM"; the same on the iitog.ru and manulx.blog
pages). The variant whose largest finite value is 448 is the OCP 8-bit
floating point specification's E4M3: 1 sign bit, 4 exponent bits with bias 7,
3 mantissa bits, no infinities, and NaN only for S.1111.111. The encoder rounds
to nearest with ties to the even code and saturates to +-448 (the reading the
build takes where the pages are silent).

Three independent formulations live here:

* ``DECODE`` -- the 256-entry value table from the bit layout (closed form).
* ``encode`` -- the definition of round-to-nearest: among the 127 non-negative
  finite codes pick the one whose value is nearest to |y|, on an exact tie the
  even code, then put y's sign bit on it. ``encode_bruteforce`` is the same
  definition evaluated literally with an argmin over all codes (slow);
  ``encode`` finds the two neighbours by binary search (fast).
* ``encode_bitlevel`` -- round-half-even of the scaled significand, written
  with frexp/rint on the exponent and mantissa fields. It shares nothing with
  ``encode`` and exists only so the two can be compared exhaustively.
"""

from __future__ import annotations

import math

import numpy as np

MAX_FINITE = 448.0
NAN_CODE = 0x7F          # S.1111.111 with S = 0; 0xFF is the negative one
MAX_CODE = 0x7E          # +448


def _decode_one(code: int) -> float:
    """Value of one E4M3 code from its bit fields (OCP OFP8, E4M3 column)."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.copysign(float("nan"), sign)
    if exp == 0:                        # subnormal: 0.mmm x 2^(1-7)
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


#: float64 value of every code 0..255 (NaN at 0x7F and 0xFF).
DECODE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)

#: magnitudes of the non-negative finite codes 0x00..0x7E; strictly increasing.
_MAG = DECODE[: MAX_CODE + 1].copy()


def decode(codes) -> np.ndarray:
    """E4M3 codes (any integer array) -> float64 values."""
    return DECODE[np.asarray(codes, dtype=np.uint8)]


def encode_bruteforce(y: float) -> int:
    """Encode one float: nearest code by exhaustive search, ties to even.

    NaN -> 0x7F with y's sign bit; |y| >= 448 (infinities included) -> 0x7E
    with y's sign bit; otherwise argmin over codes 0x00..0x7E of
    |DECODE[c] - |y||, the even code on an exact tie, then y's sign bit ORed in
    (so -0 and negative values that round to zero give 0x80).
    """
    y = float(y)
    sign = 0x80 if np.signbit(y) else 0x00
    if y != y:
        return NAN_CODE | sign
    a = abs(y)
    if a >= MAX_FINITE:
        return MAX_CODE | sign
    best, best_err = None, None
    for c in range(MAX_CODE + 1):
        err = abs(_MAG[c] - a)
        if best is None or err < best_err or (err == best_err and c % 2 == 0):
            best, best_err = c, err
    return best | sign


def encode(y) -> np.ndarray:
    """Vectorised ``encode_bruteforce``: float64 array -> uint8 codes.

    For each |y| the nearest candidates are the two codes that bracket it in
    the increasing magnitude table; the nearer wins and an exact tie goes to
    the even code.
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    sign = np.where(np.signbit(y), 0x80, 0x00).astype(np.uint8)
    nan = np.isnan(y)
    a_safe = np.where(nan, 0.0, a)
    hi = np.searchsorted(_MAG, a_safe, side="left")      # first magnitude >= a
    hi = np.clip(hi, 0, MAX_CODE)
    lo = np.clip(hi - 1, 0, MAX_CODE)
    err_hi = np.abs(_MAG[hi] - a_safe)
    err_lo = np.abs(_MAG[lo] - a_safe)
    pick = np.where(err_lo < err_hi, lo, hi)
    tie = (err_lo == err_hi) & (lo != hi)
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    pick = np.where(a_safe >= MAX_FINITE, MAX_CODE, pick)
    out = pick.astype(np.uint8) | sign
    out = np.where(nan, np.uint8(NAN_CODE) | sign, out)
    return out.astype(np.uint8)


def encode_bitlevel(y) -> np.ndarray:
    """Independent encoder: round-half-even of the significand field.

    |y| = f * 2^E with f in [0.5, 1). If |y| >= 2^-6 the code is normal with
    biased exponent E - 1 + 7 and mantissa rint((|y| / 2^(E-1) - 1) * 8); a
    mantissa of 8 carries into the exponent, which the integer sum
    (exp << 3) + man does by itself. Below 2^-6 the code is subnormal with
    mantissa rint(|y| * 2^9), where 8 again lands on the smallest normal code.
    np.rint is round-half-to-even and every scaling above is by a power of
    two, so the only rounding is the one being defined.
    """
    y = np.asarray(y, dtype=np.float64)
    sign = np.where(np.signbit(y), 0x80, 0).astype(np.int64)
    nan = np.isnan(y)
    a = np.where(nan, 0.0, np.abs(y))
    big = a >= MAX_FINITE
    a = np.where(big, 0.0, a)
    f, e = np.frexp(a)                                    # a = f * 2^e
    normal = a >= 2.0 ** -6
    man_n = np.rint((f * 2.0 - 1.0) * 8.0).astype(np.int64)
    code_n = ((e - 1 + 7).astype(np.int64) << 3) + man_n
    code_s = np.rint(a * 2.0 ** 9).astype(np.int64)
    code = np.where(normal, code_n, code_s)
    code = np.where(big, MAX_CODE, code)
    code = np.where(nan, NAN_CODE, code)
    return (code | sign).astype(np.uint8)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):          # signalling-NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def quantize(x_bf16_bits, scale) -> np.ndarray:
    """Codes for bf16 values x stored with fp32 scale s: ENC(x / s).

    The quotient is formed in float64 from the exact bf16 and fp32 operands
    (one rounding at 53 bits) and then rounded to E4M3; this equals rounding
    the exact rational x/s once. Rounding to 53 bits is monotone, so the two
    can only differ if the float64 quotient lands exactly on an E4M3 midpoint
    M (5 significant bits) while x/s != M. Write x = X 2^a (X an integer of at
    most 8 bits), s = S 2^b (at most 24 bits) and M = m 2^c (at most 5 bits).
    Then X 2^n and m S (n = a - b - c, moving the power of two to whichever
    side keeps both integral) are integers whose difference is at most
    2^(8+5+24) 2^-53 < 1 in magnitude, hence zero: x/s would be M exactly.
    (With only 24 bits, as in a plain fp32 division, the bound is 2^13 and
    the midpoint trap is real; see the tests.)
    """
    x = bf16_bits_to_f64(x_bf16_bits)
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return encode(x / s)


def dequantize(codes, scale) -> np.ndarray:
    """Dequantize on read: DECODE[code] * s in float64."""
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return decode(codes) * s
