"""Prepared calls: each decode entry point checked once (``prepare=True``) and
enqueued again from its prepared form gives, bit for bit, what the direct
calls give, while the contents of its buffers (lengths, positions, new
tokens, queries) change from step to step, as in a decode loop whose buffers
stay in place."""

import numpy as np
import pytest
import torch

import synth
from synth.device import DeviceState
from tests.gpu_harness import DEV, gpu_step, say, sm_scale_for, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kv():
    import fp8_e4m3_paged_amd as k
    k.load()
    return k


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("partition_tokens", [0, 512])
def test_prepared_calls_equal_direct_calls(kv, fused, partition_tokens):
    wl = synth.mixed_8req(max_steps=3)
    direct = DeviceState(wl, kv, device=DEV)
    prep = DeviceState(wl, kv, device=DEV)
    sm = sm_scale_for(wl)
    shape = (wl.batch, wl.num_q_heads, wl.head_dim)
    # fixed buffers whose contents each step overwrites
    seq_buf = torch.empty_like(prep.seq_lens(0))
    pos_buf = torch.empty_like(prep.tok_pos(0))
    layer_bufs = {}
    for layer in prep.layers:
        q, kn, vn = prep.step_layer_inputs(layer, 0)
        layer_bufs[layer] = (torch.empty_like(q), torch.empty_like(kn), torch.empty_like(vn),
                             torch.empty(shape, dtype=torch.float32, device=DEV))
    ws = workspace(wl, partition_tokens)
    calls = [kv.kv_verify_tags(prep.pool_tags, prep.block_table, prep.expected_tags, seq_buf,
                               prep.abort, prepare=True)]
    for layer in prep.layers:
        q, kn, vn, out = layer_bufs[layer]
        if fused:
            calls.append(kv.paged_decode_attn_append(
                q, kn, vn, prep.k_pool[layer], prep.v_pool[layer], prep.k_scale[layer],
                prep.v_scale[layer], prep.block_table, seq_buf, wl.max_seq_len, out, sm,
                workspace=ws, abort=prep.abort, partition_tokens=partition_tokens, prepare=True))
            continue
        calls.append(kv.kv_append_quant(kn, vn, prep.tok_seq, pos_buf, prep.block_table,
                                        prep.k_scale[layer], prep.v_scale[layer],
                                        prep.k_pool[layer], prep.v_pool[layer], abort=prep.abort,
                                        prepare=True))
        calls.append(kv.paged_decode_attn(q, prep.k_pool[layer], prep.v_pool[layer],
                                          prep.k_scale[layer], prep.v_scale[layer],
                                          prep.block_table, seq_buf, wl.max_seq_len, out, sm,
                                          workspace=ws, abort=prep.abort,
                                          partition_tokens=partition_tokens, prepare=True))
    assert all(isinstance(c, kv.Prepared) for c in calls)
    torch.cuda.synchronize()
    for step in range(3):
        ab_d, outs_d, _ = gpu_step(direct, step, partition_tokens=partition_tokens, fused=fused)
        seq_buf.copy_(prep.seq_lens(step))
        pos_buf.copy_(prep.tok_pos(step))
        for layer in prep.layers:
            q, kn, vn, out = layer_bufs[layer]
            sq, skn, svn = prep.step_layer_inputs(layer, step)
            q.copy_(sq)
            kn.copy_(skn)
            vn.copy_(svn)
            out.fill_(float("nan"))
        for call in calls:
            call()
        torch.cuda.synchronize()
        assert np.array_equal(prep.abort.cpu().numpy(), ab_d), f"step {step}: abort mask"
        for layer in prep.layers:
            o = layer_bufs[layer][3].cpu().numpy()
            assert np.array_equal(o, outs_d[layer], equal_nan=True), f"step {step} layer {layer}"
            assert torch.equal(prep.k_pool[layer], direct.k_pool[layer])
            assert torch.equal(prep.v_pool[layer], direct.v_pool[layer])
    say(f"prepared calls (fused={fused}, partition {partition_tokens}): 3 steps equal the "
        f"direct calls")


def test_prepared_call_keeps_its_tensors_alive(kv):
    """A prepared call holds references to its tensors, so dropping the
    caller's names does not free the memory it points at."""
    wl = synth.tiny_1req(max_steps=1)
    st = DeviceState(wl, kv, device=DEV)
    seq = st.seq_lens(0).clone()
    abort = torch.full((wl.batch,), 7, dtype=torch.uint8, device=DEV)
    call = kv.kv_verify_tags(st.pool_tags, st.block_table, st.expected_tags, seq, abort,
                             prepare=True)
    ref = abort
    del seq, abort
    torch.cuda.synchronize()
    call()
    torch.cuda.synchronize()
    assert ref.cpu().tolist() == [0] * wl.batch
