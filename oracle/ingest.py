"""Oracle for prefill ingest: per-KV-head scale calibration and the write of
whole prompts into the pool's pages.

TEST INFRASTRUCTURE (see the package docstring): never used by the product path.

Source: remio.ai/it "Il serving di modelli più piccoli di Cloudflare riduce la
memoria, ma la sicurezza diventa la prova decisiva", section "Cosa ha
cambiato Cloudflare per Kimi e GLM": prefill and decode run in separate
pools; prefill processes the incoming prompt and builds its initial cache
state, and the BF16 cache is kept where compute dominates while the smaller
FP8 form is used where memory capacity or bandwidth binds (the same page,
section "Perché le cache più piccole di Cloudflare battono la velocità pura":
prefill stays compute-bound, decode becomes memory-bound). Ingest is the
handoff of a prompt's BF16 keys and values into the FP8 decode cache.

The pages give no calibration rule, layout or page handling; the readings
taken here (each listed with its reason in the design notes) are:

* the scale of (layer, KV head) is fp32(amax / 448), where amax is the
  largest |x| over the finite bf16 values of that head's ingested tokens
  (NaN and +-Inf are skipped: they are not magnitudes of the data); amax = 0,
  or no finite value, gives 1.0, and a quotient below the smallest normal
  fp32 is raised to it, so every scale is a positive normal fp32;
* ingest writes the pages j < ceil(L / P) of every request that is not
  aborted, whole: slot t < L of page j holds token 16 j + slot's codes and the
  slots past L in the last page are set to code 0 (BF16: bits 0); a page id
  outside the pool is skipped; a request with L <= 0, with more pages than its
  table row holds, longer than the call's max_seq_len, or whose rows are not
  all inside the inputs writes nothing.
  Token t of request b is row row_start[b] + t of the packed bf16 inputs
  [rows][num_kv_heads][head_dim].
"""

from __future__ import annotations

import numpy as np

from . import e4m3

FLT_MIN = np.float32(2.0 ** -126)          # smallest normal fp32


def amax_finite(x_bits) -> np.ndarray:
    """bf16 bits [rows][num_kv_heads][head_dim] -> float32 [num_kv_heads]:
    the largest |x| over the finite values of each head (0 where none)."""
    x = np.abs(e4m3.bf16_bits_to_f64(x_bits))
    x = np.where(np.isfinite(x), x, 0.0)
    if x.shape[0] == 0:
        return np.zeros(x.shape[1], dtype=np.float32)
    return x.max(axis=(0, 2)).astype(np.float32)     # a bf16 value: exact in fp32


def scales_from_amax(amax) -> np.ndarray:
    """Per-head scale for the stored codes: fp32(amax / 448) for finite
    amax > 0, raised to the smallest normal fp32 if below it; 1.0 otherwise.

    The quotient of the two fp32 operands is formed in float64 and then
    rounded to fp32; with 53 >= 2 * 24 + 2 bits that double rounding equals
    rounding the exact quotient once (the tests also check it against exact
    rationals)."""
    with np.errstate(invalid="ignore"):           # signalling-NaN patterns stay NaN
        a = np.asarray(amax, dtype=np.float32).astype(np.float64)
        s = (a / 448.0).astype(np.float32)
    ok = np.isfinite(a) & (a > 0)
    return np.where(ok, np.maximum(s, FLT_MIN), np.float32(1.0)).astype(np.float32)


def ingest(k_pool, v_pool, k_rows, v_rows, row_start, seq_lens, block_table, cache,
           k_scale=None, v_scale=None, abort=None, max_seq_len=None):
    """Write whole prompts into the logical pools (in place); returns them.

    k_pool, v_pool: [num_pages][num_kv_heads][P][head_dim], uint8 codes (FP8)
    or uint16 bf16 bits (BF16). k_rows, v_rows: uint16 bf16 bits
    [rows][num_kv_heads][head_dim]. For each request b that is not aborted,
    with 0 < L = seq_lens[b] <= P * (table row length), and each page
    j < ceil(L / P) whose id is inside the pool:
        pool[page][g][slot][:] = code of row row_start[b] + P j + slot, head g,
                                 for P j + slot < L
        pool[page][g][slot][:] = 0 for the slots past L
    where the code is ENC(x / s_g) (FP8) or the bf16 bits unchanged (BF16).
    A request longer than max_seq_len (when given), or whose rows are not all
    inside the inputs, writes nothing.
    """
    block_table = np.asarray(block_table)
    num_pages, hkv, P, D = k_pool.shape
    batch, stride = block_table.shape
    for b in range(batch):
        L = int(seq_lens[b])
        if (abort is not None and abort[b]) or L <= 0 or -(-L // P) > stride:
            continue
        if max_seq_len is not None and L > max_seq_len:
            continue
        if int(row_start[b]) < 0 or int(row_start[b]) + L > k_rows.shape[0]:
            continue
        for j in range(-(-L // P)):
            page = int(block_table[b, j])
            if page < 0 or page >= num_pages:
                continue
            n = min(P, L - P * j)
            rows = int(row_start[b]) + P * j + np.arange(n)
            for pool, src, scale in ((k_pool, k_rows, k_scale), (v_pool, v_rows, v_scale)):
                vals = src[rows]                              # [n][hkv][D]
                if cache == "fp8":
                    codes = e4m3.quantize(vals, np.asarray(scale, np.float32)[None, :, None])
                else:
                    codes = vals
                pool[page, :, :n, :] = np.transpose(codes, (1, 0, 2))
                pool[page, :, n:, :] = 0
    return k_pool, v_pool
