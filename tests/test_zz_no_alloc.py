"""The no-alloc entry point (paged_decode_attn_append_noalloc) against the
entry point it varies (paged_decode_attn_append with a caller workspace).

Two calls in a row share the library's static scratch, the second with a
smaller input (fewer requests, other partitions), each compared with the
workspace call on identical copies of the state: outputs and pools bit for
bit, and the outputs within the attention tolerance of the oracle. Also the
persistent kernel's path (short partitions, separate reduction), the call
captured in a HIP graph and replayed with new queries, and the refusal of a
size whose workspace exceeds the scratch.
"""

import numpy as np
import pytest
import torch

import synth
from synth.device import DeviceState
from tests import helpers
from tests.gpu_harness import DEV, OracleRun, say, sm_scale_for, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kv():
    import fp8_e4m3_paged_amd as k
    k.load()
    return k


def _pair(kv, wl, rows, partition_tokens, step=0, cache="fp8"):
    """One fused call through each entry point on twin states; the requests
    ``rows`` only (a smaller batch reads a prefix of the tables)."""
    a = DeviceState(wl, kv, cache=cache, device=DEV, layers=[0])
    b = DeviceState(wl, kv, cache=cache, device=DEV, layers=[0])
    cd = kv.KV_CACHE_FP8_E4M3 if cache == "fp8" else kv.KV_CACHE_BF16
    n = len(rows)
    q, kn, vn = a.step_layer_inputs(0, step)
    q, kn, vn = q[:n].contiguous(), kn[:n].contiguous(), vn[:n].contiguous()
    seq = a.seq_lens(step)[:n].contiguous()
    bt = a.block_table[:n].contiguous()
    msl = int(wl.seq_lens_at(step)[:n].max())
    sm = sm_scale_for(wl)
    outs = []
    for st, noalloc in ((a, False), (b, True)):
        out = torch.full((n, wl.num_q_heads, wl.head_dim), float("nan"), device=DEV)
        if noalloc:
            kv.paged_decode_attn_append_noalloc(q, kn, vn, st.k_pool[0], st.v_pool[0],
                                                st.k_scale[0], st.v_scale[0], bt, seq, msl, out,
                                                sm, partition_tokens=partition_tokens,
                                                cache_dtype=cd)
        else:
            nb = kv.paged_decode_attn_workspace_bytes(n, wl.num_q_heads, wl.num_kv_heads, msl,
                                                      partition_tokens, cache_dtype=cd)
            assert nb > 0, "the case must use a workspace"
            ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
            kv.paged_decode_attn_append(q, kn, vn, st.k_pool[0], st.v_pool[0], st.k_scale[0],
                                        st.v_scale[0], bt, seq, msl, out, sm, workspace=ws,
                                        partition_tokens=partition_tokens, cache_dtype=cd)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), "outputs differ from the workspace entry point"
    assert torch.equal(a.k_pool[0], b.k_pool[0]) and torch.equal(a.v_pool[0], b.v_pool[0])
    # the oracle, for the full batch only (its tables cover every request)
    if n == wl.batch:
        orc = OracleRun(a)
        inputs = {0: (q.view(torch.int16).cpu().numpy().view(np.uint16),
                      kn.cpu().numpy().view(np.uint16), vn.cpu().numpy().view(np.uint16))}
        _, want = orc.step(step, inputs, verify=False)
        helpers.check_attention(outs[1].cpu().numpy(), want[0], label="noalloc vs oracle")
    return outs[1]


def test_noalloc_two_calls_second_smaller(kv):
    wl = synth.mixed_8req(max_steps=1)
    say("noalloc: call 1, 8 requests, automatic partitions")
    _pair(kv, wl, list(range(8)), 0)
    say("noalloc: call 2, 3 requests, 512-token partitions")
    _pair(kv, wl, [0, 1, 2], 512)


def test_noalloc_bf16_cache_two_calls_second_smaller(kv):
    """The BF16-cache variant of the no-alloc call: automatic partitions
    (sized for 2-byte elements), then a smaller call with 256-token ones."""
    wl = synth.mixed_8req(max_steps=1)
    say("noalloc bf16: call 1, 8 requests, automatic partitions")
    _pair(kv, wl, list(range(8)), 0, cache="bf16")
    say("noalloc bf16: call 2, 4 requests, 256-token partitions")
    _pair(kv, wl, [0, 1, 2, 3], 256, cache="bf16")


def test_noalloc_persistent_kernel_then_shared(kv):
    """64-token partitions run the persistent kernel (separate reduction);
    then a smaller shared-kernel call on the same scratch."""
    wl = synth.mixed_8req(max_steps=1)
    from tests import wave_split_model as ws
    assert ws.uses_wave_kernel(8, 8, wl.max_seq_len, 64)
    _pair(kv, wl, list(range(8)), 64)
    _pair(kv, wl, [0, 1], 1024)


def test_noalloc_call_captured_in_a_graph_replays_like_eager(kv):
    """A caller under graph capture: the no-alloc call (FP8, 512-token
    partitions, so the split partials live in the static scratch) captured
    once and replayed with new queries written between replays, each replay
    against the workspace entry point run eagerly on the same inputs: outputs
    bit for bit, pools equal. (The first call on the device, which looks up
    the scratch address, runs before the capture.)"""
    wl = synth.mixed_8req(max_steps=1)
    a = DeviceState(wl, kv, device=DEV, layers=[0])
    b = DeviceState(wl, kv, device=DEV, layers=[0])
    q, kn, vn = a.step_layer_inputs(0, 0)
    msl, sm, pt = wl.max_seq_len, sm_scale_for(wl), 512
    shape = (wl.batch, wl.num_q_heads, wl.head_dim)
    nb = kv.paged_decode_attn_workspace_bytes(wl.batch, wl.num_q_heads, wl.num_kv_heads, msl, pt)
    assert nb > 0, "the case must use the scratch"
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    seq_a, seq_b = a.seq_lens(0), b.seq_lens(0)
    qg = q.clone()
    out_g = torch.full(shape, float("nan"), device=DEV)

    def call_noalloc():
        kv.paged_decode_attn_append_noalloc(qg, kn, vn, b.k_pool[0], b.v_pool[0], b.k_scale[0],
                                            b.v_scale[0], b.block_table, seq_b, msl, out_g, sm,
                                            partition_tokens=pt)

    call_noalloc()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call_noalloc()
    torch.cuda.synchronize()
    out_e = torch.full(shape, float("nan"), device=DEV)
    for r in range(3):
        qr = (q.float() * (1.0 + 0.25 * r)).to(torch.bfloat16)
        qg.copy_(qr)
        out_g.fill_(float("nan"))
        out_e.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        kv.paged_decode_attn_append(qr, kn, vn, a.k_pool[0], a.v_pool[0], a.k_scale[0],
                                    a.v_scale[0], a.block_table, seq_a, msl, out_e, sm,
                                    workspace=ws, partition_tokens=pt)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {r}: output differs from the eager call"
        assert torch.equal(a.k_pool[0], b.k_pool[0]) and torch.equal(a.v_pool[0], b.v_pool[0])
    say("noalloc: 3 graph replays with new queries equal the workspace entry point")


def test_noalloc_refuses_a_workspace_beyond_its_scratch(kv):
    batch, hq, hkv, msl = 16, 64, 8, 131_073
    need = kv.paged_decode_attn_workspace_bytes(batch, hq, hkv, msl, 512)
    assert need > kv.KV_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((batch, hq, 128), dtype=torch.bfloat16, device=DEV)
    kn = torch.zeros((batch, hkv, 128), dtype=torch.bfloat16, device=DEV)
    pools = torch.zeros((4, hkv, 2048), dtype=torch.uint8, device=DEV)
    sc = torch.ones(hkv, dtype=torch.float32, device=DEV)
    bt = torch.zeros((batch, 8193), dtype=torch.int32, device=DEV)
    seq = torch.ones(batch, dtype=torch.int32, device=DEV)
    out = torch.full((batch, hq, 128), 7.0, device=DEV)
    with pytest.raises(kv.KvError) as e:
        kv.paged_decode_attn_append_noalloc(q, kn, kn, pools, pools.clone(), sc, sc, bt, seq, msl,
                                            out, 0.1, partition_tokens=512)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)                    # nothing was enqueued
