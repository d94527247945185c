"""GPU-side test harness: run decode steps through the C ABI and run the same
steps through the oracle on the host. Imported by the GPU tests only."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import fp8_e4m3_paged_amd as kv
from oracle import paged
from synth.device import DeviceState
from tests import helpers

DEV = "cuda"


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def sm_scale_for(wl) -> float:
    return 1.0 / math.sqrt(wl.head_dim)


def workspace(wl, partition_tokens: int, max_seq_len=None):
    """A zero-filled workspace that fits either cache's partitioning."""
    n = max(kv.paged_decode_attn_workspace_bytes(wl.batch, wl.num_q_heads, wl.num_kv_heads,
                                                 max_seq_len or wl.max_seq_len, partition_tokens,
                                                 cache_dtype=cd)
            for cd in (kv.KV_CACHE_FP8_E4M3, kv.KV_CACHE_BF16))
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=DEV) if n else None


def verify_workspace(st: DeviceState):
    """Zeroed counters for the split tag check, or None when every row fits one chunk."""
    n = kv.kv_verify_tags_workspace_bytes(st.wl.batch, st.block_table.shape[1])
    return torch.zeros(n, dtype=torch.uint8, device=DEV) if n else None


def gpu_step(st: DeviceState, step: int, verify: bool = True, partition_tokens: int = 0,
             sm_scale=None, layers=None, max_seq_len=None, fused: bool = False):
    """One decode step on the GPU (separate append + attention calls, or the
    fused paged_decode_attn_append). Returns (abort or None, {layer: out},
    {layer: (q, kn, vn)})."""
    wl = st.wl
    layers = st.layers if layers is None else layers
    sm = sm_scale_for(wl) if sm_scale is None else sm_scale
    msl = max_seq_len or wl.max_seq_len
    seq_lens = st.seq_lens(step)
    tok_pos = st.tok_pos(step)
    ws = workspace(wl, partition_tokens, msl)
    abort = None
    if verify:
        kv.kv_verify_tags(st.pool_tags, st.block_table, st.expected_tags, seq_lens, st.abort,
                          workspace=verify_workspace(st))
        abort = st.abort
    outs, inputs = {}, {}
    for layer in layers:
        q, kn, vn = st.step_layer_inputs(layer, step)
        cd = kv.KV_CACHE_FP8_E4M3 if st.cache == "fp8" else kv.KV_CACHE_BF16
        if fused:
            out = torch.full((wl.batch, wl.num_q_heads, wl.head_dim), float("nan"),
                             dtype=torch.float32, device=DEV)
            kv.paged_decode_attn_append(q, kn, vn, st.k_pool[layer], st.v_pool[layer],
                                        st.k_scale[layer], st.v_scale[layer], st.block_table,
                                        seq_lens, msl, out, sm, workspace=ws, abort=abort,
                                        partition_tokens=partition_tokens, cache_dtype=cd)
            outs[layer] = out
            inputs[layer] = (q.view(torch.int16).cpu().numpy().view(np.uint16),
                             kn.cpu().numpy().view(np.uint16), vn.cpu().numpy().view(np.uint16))
            continue
        if st.cache == "fp8":
            kv.kv_append_quant(kn, vn, st.tok_seq, tok_pos, st.block_table, st.k_scale[layer],
                               st.v_scale[layer], st.k_pool[layer], st.v_pool[layer],
                               abort=abort)
        else:
            kv.kv_append_bf16(kn, vn, st.tok_seq, tok_pos, st.block_table, st.k_pool[layer],
                              st.v_pool[layer], abort=abort)
        out = torch.full((wl.batch, wl.num_q_heads, wl.head_dim), float("nan"),
                         dtype=torch.float32, device=DEV)
        kv.paged_decode_attn(q, st.k_pool[layer], st.v_pool[layer], st.k_scale[layer],
                             st.v_scale[layer], st.block_table, seq_lens, msl, out, sm,
                             workspace=ws, abort=abort, partition_tokens=partition_tokens,
                             cache_dtype=kv.KV_CACHE_FP8_E4M3 if st.cache == "fp8"
                             else kv.KV_CACHE_BF16)
        outs[layer] = out
        inputs[layer] = (q.view(torch.int16).cpu().numpy().view(np.uint16),
                         kn.cpu().numpy().view(np.uint16), vn.cpu().numpy().view(np.uint16))
    torch.cuda.synchronize()
    ab = st.abort.cpu().numpy().copy() if verify else None
    return ab, {k: v.cpu().numpy() for k, v in outs.items()}, inputs


def device_pool_logical(st: DeviceState, layer: int):
    """The GPU pools of one layer as logical [pages][Hkv][16][128] host arrays."""
    kt = st.k_pool[layer].cpu().numpy()
    vt = st.v_pool[layer].cpu().numpy()
    if st.cache == "bf16":
        kt, vt = kt.view(np.uint16), vt.view(np.uint16)
    return (helpers.tiles_to_logical(kt, "k", st.cache),
            helpers.tiles_to_logical(vt, "v", st.cache))


class OracleRun:
    """The oracle's copy of a whole (small) workload: pools per layer on the host."""

    def __init__(self, st: DeviceState):
        self.st = st
        wl = st.wl
        self.kp, self.vp = {}, {}
        for layer in st.layers:
            self.kp[layer], self.vp[layer] = helpers.oracle_pools(
                wl, layer, st.k_scale_host[layer], st.v_scale_host[layer], st.cache)

    def step(self, step: int, inputs, verify=True, sm_scale=None):
        """The oracle's decode step (paged.decode_step) over the layers in
        ``inputs`` ({layer: (q, k_new, v_new)} bf16 bits), updating the host
        pools in place. Returns (abort or None without the check, {layer: out})."""
        st, wl = self.st, self.st.wl
        layers = list(inputs)
        state = dict(pool_tags=wl.pool_tags, block_table=wl.block_table,
                     expected_tags=wl.expected_tags, seq_lens=wl.seq_lens_at(step),
                     page_size=wl.page_size,
                     k_pool=[self.kp[ly] for ly in layers], v_pool=[self.vp[ly] for ly in layers],
                     k_scale=[st.k_scale_host[ly] for ly in layers],
                     v_scale=[st.v_scale_host[ly] for ly in layers])
        sm = sm_scale_for(wl) if sm_scale is None else sm_scale
        abort, outs = paged.decode_step(state, [inputs[ly][0] for ly in layers],
                                        [inputs[ly][1] for ly in layers],
                                        [inputs[ly][2] for ly in layers], sm, cache=st.cache,
                                        verify=verify)
        return (abort if verify else None), dict(zip(layers, outs))


def oracle_request(st: DeviceState, layer: int, b: int, step: int, q_bits, sm_scale=None):
    """Oracle output [Hq][D] of one request of a large workload, regenerated alone.

    The request's pool content is the initial tokens plus the tokens appended at
    steps 0..step, all defined by the seeded generator, quantized by the oracle.
    Also returns the oracle's codes so the caller can compare the GPU's pages.
    """
    wl = st.wl
    L = int(wl.seq_lens_at(step)[b])
    kc, vc = helpers.request_codes(wl, layer, b, L, st.k_scale_host[layer],
                                   st.v_scale_host[layer], st.cache)
    sm = sm_scale_for(wl) if sm_scale is None else sm_scale
    if st.cache == "fp8":
        Kd = paged.e4m3.dequantize(kc, st.k_scale_host[layer][:, None, None])
        Vd = paged.e4m3.dequantize(vc, st.v_scale_host[layer][:, None, None])
    else:
        Kd = paged.e4m3.bf16_bits_to_f64(kc)
        Vd = paged.e4m3.bf16_bits_to_f64(vc)
    return paged.attend_request(q_bits[b], Kd, Vd, sm), kc, vc
