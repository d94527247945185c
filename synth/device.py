"""Device-side construction of a workload's state (test and benchmark harness).

The same integer hash as ``synth`` evaluated with torch int64 ops on the GPU,
so a multi-GB pool is generated in place with exactly the bits the host would
produce for any single request. Pools are then filled through the library's
own bulk append (``kv_append_quant`` / ``kv_append_bf16``): the prefill-ingest
use of the append entry points.

This module holds no E4M3, tag-check or attention arithmetic.
"""

from __future__ import annotations

import numpy as np
import torch

from . import M32, Workload, normal_table, scales_from_amax

_C1 = 0x85EBCA6B
_C2 = 0xC2B2AE35


def _mul32(h: torch.Tensor, c: int) -> torch.Tensor:
    lo, hi = c & 0xFFFF, c >> 16
    return (h * lo + (((h * hi) & 0xFFFF) << 16)) & M32


def fmix32(h: torch.Tensor) -> torch.Tensor:
    h = h ^ (h >> 16)
    h = _mul32(h, _C1)
    h = h ^ (h >> 13)
    h = _mul32(h, _C2)
    return h ^ (h >> 16)


def table_index(k1: torch.Tensor, k2: torch.Tensor, ctr: torch.Tensor) -> torch.Tensor:
    """Device twin of ``synth.table_index`` (k1, k2 broadcast against ctr)."""
    h = fmix32(ctr ^ k1)
    h = fmix32((h + k2) & M32)
    return h >> 16


_TABLES: dict = {}


def device_table(sigma: float, device) -> torch.Tensor:
    key = (sigma, str(device))
    if key not in _TABLES:
        _TABLES[key] = torch.from_numpy(normal_table(sigma).view(np.int16)).to(device)
    return _TABLES[key]


def _keys(wl: Workload, layer: int, kind: str, device) -> tuple[torch.Tensor, torch.Tensor]:
    ks = [wl._kv_key(layer, kind, b) for b in range(wl.batch)]
    k1 = torch.tensor([k[0] for k in ks], dtype=torch.int64, device=device)
    k2 = torch.tensor([k[1] for k in ks], dtype=torch.int64, device=device)
    return k1, k2


def kv_bits_tokens(wl: Workload, layer: int, kind: str, tok_seq: torch.Tensor,
                   tok_pos: torch.Tensor, keys=None) -> torch.Tensor:
    """bf16 bits (int16) [n][Hkv][D] of tokens (tok_seq[n], tok_pos[n])."""
    dev = tok_seq.device
    hkv, d = wl.num_kv_heads, wl.head_dim
    k1, k2 = keys if keys is not None else _keys(wl, layer, kind, dev)
    seq = tok_seq.to(torch.int64)
    ctr = (tok_pos.to(torch.int64)[:, None, None] * hkv
           + torch.arange(hkv, device=dev, dtype=torch.int64)[None, :, None]) * d \
        + torch.arange(d, device=dev, dtype=torch.int64)[None, None, :]
    idx = table_index(k1[seq][:, None, None], k2[seq][:, None, None], ctr)
    return device_table(wl.kv_sigma(kind), dev)[idx]


def _token_chunks(wl: Workload, chunk_tokens: int, device):
    """(tok_seq, tok_pos) chunks covering every initial token of every request."""
    seqs, poss = [], []
    for b in range(wl.batch):
        L = int(wl.seq_lens0[b])
        seqs.append(np.full(L, b, dtype=np.int32))
        poss.append(np.arange(L, dtype=np.int32))
    seq = np.concatenate(seqs) if seqs else np.zeros(0, np.int32)
    pos = np.concatenate(poss) if poss else np.zeros(0, np.int32)
    for i in range(0, len(seq), chunk_tokens):
        yield (torch.from_numpy(seq[i:i + chunk_tokens]).to(device),
               torch.from_numpy(pos[i:i + chunk_tokens]).to(device))


def prompt_rows(wl: Workload, layer: int, kind: str, device="cuda", chunk_tokens: int = 65536):
    """Every request's initial tokens packed request by request: bf16 bits
    (int16) [sum L0][Hkv][D] and the int32 row where each request starts."""
    keys = _keys(wl, layer, kind, device)
    parts = [kv_bits_tokens(wl, layer, kind, seq, pos, keys)
             for seq, pos in _token_chunks(wl, chunk_tokens, device)]
    rows = (torch.cat(parts) if parts else
            torch.zeros((0, wl.num_kv_heads, wl.head_dim), dtype=torch.int16, device=device))
    lens = wl.seq_lens0.astype(np.int64)
    start = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    return rows, torch.from_numpy(start).to(device)


def device_amax(wl: Workload, layer: int, chunk_tokens: int = 32768, device="cuda"):
    """Per-KV-head amax of |K| and |V| over the initial pool (exact: max of bf16)."""
    out = []
    for kind in ("k", "v"):
        keys = _keys(wl, layer, kind, device)
        amax = torch.zeros(wl.num_kv_heads, dtype=torch.float32, device=device)
        for seq, pos in _token_chunks(wl, chunk_tokens, device):
            vals = kv_bits_tokens(wl, layer, kind, seq, pos, keys).view(torch.bfloat16)
            amax = torch.maximum(amax, vals.abs().amax(dim=(0, 2)).float())
        out.append(amax.cpu().numpy())
    return out[0], out[1]


class DeviceState:
    """Device tensors of one workload: tables, tags, per-layer pools and scales.

    ``cache`` is "fp8" or "bf16". Pools hold the initial tokens of every
    request after construction; each decode step appends one token per
    request. ``scales`` may be given (host fp32 arrays per layer) or are
    computed as amax / 448 from the device-generated values.
    """

    def __init__(self, wl: Workload, lib, cache: str = "fp8", device="cuda",
                 layers=None, chunk_tokens: int = 32768, scales=None, fill=True):
        self.wl = wl
        self.cache = cache
        self.device = device
        self.layers = list(range(wl.num_layers)) if layers is None else list(layers)
        self.block_table = torch.from_numpy(wl.block_table).to(device)
        self.pool_tags = torch.from_numpy(wl.pool_tags.view(np.int32)).to(device)
        self.expected_tags = torch.from_numpy(wl.expected_tags.view(np.int32)).to(device)
        self.seq_lens0 = torch.from_numpy(wl.seq_lens0.astype(np.int32)).to(device)
        self.tok_seq = torch.arange(wl.batch, dtype=torch.int32, device=device)
        self.abort = torch.zeros(wl.batch, dtype=torch.uint8, device=device)
        tile = 16 * wl.head_dim   # elements per (page, head) tile: u8 codes or int16 bf16 bits
        pool_dtype = torch.uint8 if cache == "fp8" else torch.int16
        self.k_pool, self.v_pool, self.k_scale, self.v_scale = {}, {}, {}, {}
        self.k_scale_host, self.v_scale_host = {}, {}
        for layer in self.layers:
            shape = (wl.num_pages, wl.num_kv_heads, tile)
            self.k_pool[layer] = torch.zeros(shape, dtype=pool_dtype, device=device)
            self.v_pool[layer] = torch.zeros(shape, dtype=pool_dtype, device=device)
            if scales is not None:
                ks, vs = scales[layer]
            elif cache == "fp8":
                ka, va = device_amax(wl, layer, chunk_tokens, device)
                ks, vs = scales_from_amax(ka), scales_from_amax(va)
            else:
                ks = vs = np.ones(wl.num_kv_heads, dtype=np.float32)
            self.k_scale_host[layer] = np.asarray(ks, dtype=np.float32)
            self.v_scale_host[layer] = np.asarray(vs, dtype=np.float32)
            self.k_scale[layer] = torch.from_numpy(self.k_scale_host[layer]).to(device)
            self.v_scale[layer] = torch.from_numpy(self.v_scale_host[layer]).to(device)
            if fill:
                self.fill_layer(lib, layer, chunk_tokens)

    def fill_layer(self, lib, layer: int, chunk_tokens: int = 32768):
        """Write every initial token of every request through the bulk append."""
        wl = self.wl
        kk = _keys(wl, layer, "k", self.device)
        vk = _keys(wl, layer, "v", self.device)
        for seq, pos in _token_chunks(wl, chunk_tokens, self.device):
            k = kv_bits_tokens(wl, layer, "k", seq, pos, kk)
            v = kv_bits_tokens(wl, layer, "v", seq, pos, vk)
            if self.cache == "fp8":
                lib.kv_append_quant(k, v, seq, pos, self.block_table, self.k_scale[layer],
                                    self.v_scale[layer], self.k_pool[layer], self.v_pool[layer])
            else:
                lib.kv_append_bf16(k, v, seq, pos, self.block_table, self.k_pool[layer],
                                   self.v_pool[layer])

    # ---- per-step inputs --------------------------------------------------
    def seq_lens(self, step: int) -> torch.Tensor:
        return self.seq_lens0 + (step + 1)

    def tok_pos(self, step: int) -> torch.Tensor:
        return self.seq_lens0 + step

    def upload_tags(self):
        self.pool_tags.copy_(torch.from_numpy(self.wl.pool_tags.view(np.int32)))
        self.expected_tags.copy_(torch.from_numpy(self.wl.expected_tags.view(np.int32)))

    def step_layer_inputs(self, layer: int, step: int):
        """q, k_new, v_new of one layer and step (host-generated, uploaded)."""
        wl = self.wl
        q = torch.from_numpy(wl.q_bits(layer, step).view(np.int16)).to(self.device)
        kn = torch.from_numpy(wl.new_token_bits(layer, "k", step).view(np.int16)).to(self.device)
        vn = torch.from_numpy(wl.new_token_bits(layer, "v", step).view(np.int16)).to(self.device)
        return q.view(torch.bfloat16), kn, vn


def q_bits_device(wl: Workload, layer: int, step: int, device="cuda") -> torch.Tensor:
    """Device twin of ``Workload.q_bits``: bf16 [B][Hq][D] decode queries."""
    from . import T_Q, stream_key
    k1, k2 = stream_key(wl.seed, T_Q, layer, step)
    n = wl.batch * wl.num_q_heads * wl.head_dim
    ctr = torch.arange(n, dtype=torch.int64, device=device)
    idx = table_index(torch.tensor(k1, device=device), torch.tensor(k2, device=device), ctr)
    bits = device_table(wl.q_sigma, device)[idx]
    return bits.view(wl.batch, wl.num_q_heads, wl.head_dim).view(torch.bfloat16)


def new_token_bits_device(wl: Workload, layer: int, kind: str, step: int,
                          device="cuda") -> torch.Tensor:
    """Device twin of ``Workload.new_token_bits``: int16 [B][Hkv][D]."""
    seq = torch.arange(wl.batch, dtype=torch.int32, device=device)
    pos = torch.from_numpy((wl.seq_lens0 + step).astype(np.int32)).to(device)
    return kv_bits_tokens(wl, layer, kind, seq, pos)
