"""Oracle for the paged decode step: tag check, quantize-on-append, attention.

TEST INFRASTRUCTURE (see the package docstring): never used by the product path.

Everything here works on the *logical* pool layout

    k_pool, v_pool : [num_pages][num_kv_heads][page_size][head_dim]
                     uint8 E4M3 codes (FP8 cache) or uint16 bf16 bits (BF16 cache)

and plain integer tables

    block_table    : int32  [batch][max_pages]   logical page j -> physical page
    expected_tags  : uint32 [batch][max_pages]   tag the request expects there
    pool_tags      : uint32 [num_pages]          current tag of each physical page
    seq_lens       : int32  [batch]              tokens attended, appended one included

Sources (the five pages report one Cloudflare post; titles as printed):

* page-tag check -- remio.ai/it "Il serving di modelli più piccoli di
  Cloudflare riduce la memoria, ma la sicurezza diventa la prova decisiva",
  sections "Cosa ha cambiato Cloudflare per Kimi e GLM" (every physical page
  has a tag that changes on reallocation; the server records each request's
  expected pages and tags; a mismatch aborts that request before supported
  decode ops read) and "La sicurezza della cache KV condivisa diventa una
  questione di produzione" (the validation runs as a separate batched check;
  a no-op tracker exists where it is disabled). Same on iitog.ru and
  manulx.blog ("共有キャッシュの保護").
* FP8 cache and dequantize-on-read -- remio.ai/it, sections "Cosa ha cambiato
  ..." (K/V stored in FP8 e4m3 instead of BF16) and "Perché le cache più
  piccole di Cloudflare battono la velocità pura" (conversion work happens
  when the attention kernel reads cached values).
* attention itself is standard softmax attention for one decode token; the
  pages do not restate it, so the oracle is its plain definition.

Readings where the pages are silent (each is listed with its reason in the
design notes): the tag check covers logical pages j < ceil(L/page_size),
the appended token's page included, and an out-of-range page id or a length
the table cannot hold also aborts; aborted requests are neither written by
append nor read by attention and their output is all zeros; a request with
L <= 0 attends to nothing and outputs zeros; query head h reads KV head
h // (Hq / Hkv).
"""

from __future__ import annotations

import numpy as np

from . import e4m3


def _pages_needed(L: int, page_size: int) -> int:
    return (int(L) + page_size - 1) // page_size


def verify_tags(pool_tags, block_table, expected_tags, seq_lens, page_size):
    """Batched page-tag check -> abort flags uint8[batch] (0 or 1).

    abort[b] = 1 iff some logical page j < ceil(L_b / page_size) maps to a
    physical id outside [0, num_pages) or to a page whose current tag differs
    from the tag the request recorded for it. A negative length, or one the
    request's table row cannot hold, also aborts. Entries past the request's
    last page are never looked at.
    """
    pool_tags = np.asarray(pool_tags, dtype=np.uint32)
    block_table = np.asarray(block_table, dtype=np.int64)
    expected_tags = np.asarray(expected_tags, dtype=np.uint32)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    num_pages = pool_tags.shape[0]
    batch = seq_lens.shape[0]
    max_pages = block_table.shape[1]
    abort = np.zeros(batch, dtype=np.uint8)
    for b in range(batch):
        L = int(seq_lens[b])
        if L < 0 or _pages_needed(L, page_size) > max_pages:
            abort[b] = 1
            continue
        for j in range(_pages_needed(L, page_size)):
            page = int(block_table[b, j])
            if page < 0 or page >= num_pages or pool_tags[page] != expected_tags[b, j]:
                abort[b] = 1
                break
    return abort


def _target(b, t, block_table, num_pages, page_size):
    """Physical (page, slot) for token t of request b, or None if unmapped."""
    if t < 0:
        return None
    j = t // page_size
    if j >= block_table.shape[1]:
        return None
    page = int(block_table[b, j])
    if page < 0 or page >= num_pages:
        return None
    return page, t % page_size


def append_fp8(k_pool, v_pool, k_new_bits, v_new_bits, tok_seq, tok_pos,
               block_table, k_scale, v_scale, abort=None):
    """Quantize-on-append into an FP8 pool (in place); returns the pools.

    For each new token n of request b = tok_seq[n] at position t = tok_pos[n]
    that is not aborted: page = block_table[b][t // P], slot = t % P, and for
    every KV head g

        k_pool[page][g][slot][:] = ENC(k_new[n][g][:] / s_K[g])

    and the same for V with s_V. Tokens of aborted requests, of a request
    index outside the batch, or whose target is unmapped write nothing.
    """
    block_table = np.asarray(block_table)
    num_pages, _, page_size, _ = k_pool.shape
    batch = block_table.shape[0]
    k_scale = np.asarray(k_scale, dtype=np.float32)
    v_scale = np.asarray(v_scale, dtype=np.float32)
    for n in range(len(tok_seq)):
        b, t = int(tok_seq[n]), int(tok_pos[n])
        if b < 0 or b >= batch or (abort is not None and abort[b]):
            continue
        tgt = _target(b, t, block_table, num_pages, page_size)
        if tgt is None:
            continue
        page, slot = tgt
        k_pool[page, :, slot, :] = e4m3.quantize(k_new_bits[n], k_scale[:, None])
        v_pool[page, :, slot, :] = e4m3.quantize(v_new_bits[n], v_scale[:, None])
    return k_pool, v_pool


def append_bf16(k_pool, v_pool, k_new_bits, v_new_bits, tok_seq, tok_pos,
                block_table, abort=None):
    """BF16-cache append: the same addressing, the value stored unchanged."""
    block_table = np.asarray(block_table)
    num_pages, _, page_size, _ = k_pool.shape
    batch = block_table.shape[0]
    for n in range(len(tok_seq)):
        b, t = int(tok_seq[n]), int(tok_pos[n])
        if b < 0 or b >= batch or (abort is not None and abort[b]):
            continue
        tgt = _target(b, t, block_table, num_pages, page_size)
        if tgt is None:
            continue
        page, slot = tgt
        k_pool[page, :, slot, :] = k_new_bits[n]
        v_pool[page, :, slot, :] = v_new_bits[n]
    return k_pool, v_pool


def gather_request(pool, block_table_row, L, page_size):
    """Logical [Hkv][L][D] view of one request's first L tokens (a copy)."""
    n = _pages_needed(L, page_size)
    pages = pool[np.asarray(block_table_row[:n], dtype=np.int64)]   # [n][Hkv][P][D]
    hkv, d = pages.shape[1], pages.shape[3]
    seq = pages.transpose(1, 0, 2, 3).reshape(hkv, n * page_size, d)
    return seq[:, :L, :]


def dequant_request(pool, block_table_row, L, page_size, scale, cache):
    """float64 [Hkv][L][D] values of one request as attention reads them."""
    raw = gather_request(pool, block_table_row, L, page_size)
    if cache == "fp8":
        return e4m3.dequantize(raw, np.asarray(scale, dtype=np.float32)[:, None, None])
    if cache == "bf16":
        return e4m3.bf16_bits_to_f64(raw)
    raise ValueError(cache)


def request_is_readable(block_table_row, L, page_size, num_pages):
    """True iff every page the first L tokens live on is a valid pool page."""
    n = _pages_needed(L, page_size)
    if n > len(block_table_row):
        return False
    ids = np.asarray(block_table_row[:n], dtype=np.int64)
    return bool(np.all((ids >= 0) & (ids < num_pages)))


def attend_request(q_bits_b, Kd, Vd, sm_scale):
    """Softmax attention of one decode token per query head, float64.

    q_bits_b: bf16 bits [Hq][D]; Kd, Vd: float64 [Hkv][L][D]. Query head h
    uses KV head g = h // (Hq / Hkv). For each h:
        s_j = (q_h . K_j) * sm_scale,   p = softmax(s),   out_h = sum_j p_j V_j
    with the softmax taken after subtracting max_j s_j.
    """
    q = e4m3.bf16_bits_to_f64(q_bits_b)
    hq = q.shape[0]
    hkv = Kd.shape[0]
    group = hq // hkv
    out = np.zeros((hq, Kd.shape[2]), dtype=np.float64)
    for g in range(hkv):
        qg = q[g * group:(g + 1) * group]                 # [G][D]
        s = (qg @ Kd[g].T) * float(sm_scale)              # [G][L]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[g * group:(g + 1) * group] = p @ Vd[g]
    return out


def decode_attn_request(b, q_bits, k_pool, v_pool, k_scale, v_scale, block_table,
                        seq_lens, sm_scale, cache="fp8", abort=None):
    """Output float64 [Hq][D] of request b (zeros if aborted / empty / unmapped)."""
    hq, d = q_bits.shape[1], q_bits.shape[2]
    num_pages, _, page_size, _ = k_pool.shape
    L = int(seq_lens[b])
    zero = np.zeros((hq, d), dtype=np.float64)
    if (abort is not None and abort[b]) or L <= 0:
        return zero
    if not request_is_readable(block_table[b], L, page_size, num_pages):
        return zero
    Kd = dequant_request(k_pool, block_table[b], L, page_size, k_scale, cache)
    Vd = dequant_request(v_pool, block_table[b], L, page_size, v_scale, cache)
    return attend_request(q_bits[b], Kd, Vd, sm_scale)


def decode_attn(q_bits, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens,
                sm_scale, cache="fp8", abort=None):
    """Decode attention for the whole batch -> float64 [batch][Hq][D]."""
    batch = q_bits.shape[0]
    return np.stack([
        decode_attn_request(b, q_bits, k_pool, v_pool, k_scale, v_scale,
                            block_table, seq_lens, sm_scale, cache, abort)
        for b in range(batch)
    ])


def decode_step(state, layers_q_bits, layers_k_new, layers_v_new, sm_scale,
                cache="fp8", verify=True):
    """One decode step over all layers, in the order the pages require.

    ``state`` is a dict with pool_tags, block_table, expected_tags, seq_lens
    (lengths *after* this step's append), page_size, and per-layer lists
    k_pool, v_pool, k_scale, v_scale (mutated in place by the append).
    Returns (abort, [out per layer]). With verify=False no check runs (the
    no-op tracker) and nothing is aborted.
    """
    P = state["page_size"]
    seq_lens = np.asarray(state["seq_lens"])
    batch = seq_lens.shape[0]
    if verify:
        abort = verify_tags(state["pool_tags"], state["block_table"],
                            state["expected_tags"], seq_lens, P)
    else:
        abort = np.zeros(batch, dtype=np.uint8)
    tok_seq = np.arange(batch)
    tok_pos = seq_lens - 1
    outs = []
    for layer in range(len(state["k_pool"])):
        if cache == "fp8":
            append_fp8(state["k_pool"][layer], state["v_pool"][layer],
                       layers_k_new[layer], layers_v_new[layer], tok_seq, tok_pos,
                       state["block_table"], state["k_scale"][layer],
                       state["v_scale"][layer], abort)
        else:
            append_bf16(state["k_pool"][layer], state["v_pool"][layer],
                        layers_k_new[layer], layers_v_new[layer], tok_seq, tok_pos,
                        state["block_table"], abort)
        outs.append(decode_attn(layers_q_bits[layer], state["k_pool"][layer],
                                state["v_pool"][layer], state["k_scale"][layer],
                                state["v_scale"][layer], state["block_table"],
                                seq_lens, sm_scale, cache, abort))
    return abort, outs
