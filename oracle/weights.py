"""Oracle for weight-only quantized decode GEMV (INT4 and FP8 e4m3 weights).

TEST INFRASTRUCTURE (see the package docstring): never used by the product path.

Source: remio.ai/it "Il serving di modelli più piccoli di Cloudflare riduce la
memoria, ma la sicurezza diventa la prova decisiva", section "La compressione
dei pesi GLM modifica il compromesso tra le fasi": GLM's weights go from FP8
to INT4; decode streams the weights from HBM again and again, so when memory
bandwidth binds, fewer bytes give each token sooner; the INT4 weights have to
be expanded before the matrix product (which is what costs prefill). The
page compares FP8 and INT4 decode throughput at 1 to 64 requests.

The page gives no number format beyond "four-bit integer" and no grouping;
the readings taken here (listed with their reasons in the design notes):

* weights W [N][K] (output row n, input k) in bf16 are quantized per row and
  per group of G = 128 consecutive k with one fp32 scale each;
* INT4: symmetric, codes q in [-8, 7], s = fp32(amax / 7) of the group's
  |w| (1.0 for an all-zero group), q = clamp(round-half-even(w / s), -8, 7)
  with the exact quotient;
* FP8 (the baseline the page compares against): E4M3 codes with
  s = fp32(amax / 448) per group and the same encoder as the KV cache;
* the product for bf16 activations X [M][K]:
      Y[m][n] = sum_k X[m][k] * q[n][k] * s[n][k // G]      (float64 here).
"""

from __future__ import annotations

import numpy as np

from . import e4m3

GROUP = 128


def _groups(w_bits, group):
    w = e4m3.bf16_bits_to_f64(w_bits)
    n, k = w.shape
    assert k % group == 0
    return w.reshape(n, k // group, group)


def _scale(amax, qmax):
    """fp32(amax / qmax), 1.0 where amax is 0 (double rounding from float64 is
    innocuous for a quotient of fp32 values: 53 >= 2 * 24 + 2)."""
    s = (amax / qmax).astype(np.float32)
    return np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)


def quantize_int4(w_bits, group=GROUP):
    """bf16 bits [N][K] -> (codes int8 [N][K] in [-8, 7], scales fp32 [N][K/G])."""
    w = _groups(w_bits, group)
    amax = np.abs(w).max(axis=2)
    s = _scale(amax, 7.0)
    q = np.rint(w / s.astype(np.float64)[:, :, None])        # float64 quotient, half to even
    q = np.clip(q, -8, 7).astype(np.int8)
    return q.reshape(w_bits.shape), s


def quantize_fp8(w_bits, group=GROUP):
    """bf16 bits [N][K] -> (E4M3 codes uint8 [N][K], scales fp32 [N][K/G])."""
    w = _groups(w_bits, group)
    s = _scale(np.abs(w).max(axis=2), 448.0)
    n, k = w_bits.shape
    codes = e4m3.quantize(np.asarray(w_bits).reshape(n, k // group, group), s[:, :, None])
    return codes.reshape(n, k), s


def dequant_int4(q, s, group=GROUP):
    n, k = q.shape
    return (q.astype(np.float64).reshape(n, k // group, group)
            * s.astype(np.float64)[:, :, None]).reshape(n, k)


def dequant_fp8(codes, s, group=GROUP):
    n, k = codes.shape
    return (e4m3.decode(codes).reshape(n, k // group, group)
            * s.astype(np.float64)[:, :, None]).reshape(n, k)


def gemv(x_bits, w_deq):
    """Y = X W^T in float64: X bf16 bits [M][K], W dequantized [N][K] -> [M][N]."""
    return e4m3.bf16_bits_to_f64(x_bits) @ w_deq.T
