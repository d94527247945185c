"""GPU tests of whole steps and of the corners of the fused headline path.

* The binding's ``decode_step`` helper (fused and separate launches) against
  the oracle's step (``oracle.paged.decode_step``) on a three-layer batch with
  a stale tag: abort mask and every pool byte bit for bit, outputs within the
  tolerance, for several steps in a row.
* Every bf16 bit pattern (NaN, infinities, values far beyond 448 s) through
  the fused append + attention launch as new tokens, in the shared and the
  persistent kernel: the codes it stores equal the oracle's.
* The prefill handoff enqueued on a side stream equals the same handoff on
  the current stream, bit for bit.
* Prepared calls while the lengths grow step by step, within the
  max_seq_len they were prepared with.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import e4m3
from synth.device import DeviceState, prompt_rows
from tests import helpers
from tests.gpu_harness import DEV, OracleRun, device_pool_logical, say, sm_scale_for, workspace
from tests.test_gpu_parity import _encode_scales

pytestmark = pytest.mark.gpu
P = 16


@pytest.fixture(scope="module")
def kv():
    import fp8_e4m3_paged_amd as k
    k.load()
    return k


def _three_layer_workload(max_steps):
    """5 requests of 1 to 700 tokens, 24 query / 4 KV heads (group 6), three
    layers, a 2x shuffled pool, one stale tag."""
    rng = np.random.default_rng(3030)
    wl = synth._build("three_layers", 30, batch=5, layers=3, hq=24, hkv=4, d=128, page=16,
                      seq_lens0=[0, 15, 300, 699, 130], max_steps=max_steps,
                      pool_pages=lambda total: 2 * total, k_sigma=1.0, v_sigma=0.5,
                      q_sigma=1.0, garbage_tail=True, rng=rng)
    p = int(wl.block_table[3, 7])
    wl.pool_tags[p] = np.uint32((int(wl.pool_tags[p]) + 1) & 0xFFFFFFFF)
    wl.stale = (3,)
    return wl


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("partition_tokens", [0, 64])
def test_binding_decode_step_against_oracle_step(kv, fused, partition_tokens):
    wl = _three_layer_workload(max_steps=3)
    st = DeviceState(wl, kv, cache="fp8", device=DEV)
    orc = OracleRun(st)
    ws = workspace(wl, partition_tokens)
    for step in range(3):
        seq = st.seq_lens(step)
        layers, inputs = [], {}
        for layer in st.layers:
            q, kn, vn = st.step_layer_inputs(layer, step)
            out = torch.full((wl.batch, wl.num_q_heads, wl.head_dim), float("nan"), device=DEV)
            layers.append(dict(q=q, k_new=kn, v_new=vn, k_pool=st.k_pool[layer],
                               v_pool=st.v_pool[layer], k_scale=st.k_scale[layer],
                               v_scale=st.v_scale[layer], out=out))
            inputs[layer] = (q.view(torch.int16).cpu().numpy().view(np.uint16),
                             kn.cpu().numpy().view(np.uint16), vn.cpu().numpy().view(np.uint16))
        kv.decode_step(layers, st.block_table, seq, st.tok_pos(step), st.tok_seq,
                       wl.max_seq_len, sm_scale_for(wl), pool_tags=st.pool_tags,
                       expected_tags=st.expected_tags, abort=st.abort, workspace=ws,
                       partition_tokens=partition_tokens, fused=fused)
        torch.cuda.synchronize()
        ab_o, outs_o = orc.step(step, inputs)
        ab = st.abort.cpu().numpy()
        assert np.array_equal(ab, ab_o) and ab.tolist() == [0, 0, 0, 1, 0]
        for i, layer in enumerate(st.layers):
            kd, vd = device_pool_logical(st, layer)
            assert np.array_equal(kd, orc.kp[layer]), f"step {step} layer {layer}: K pool"
            assert np.array_equal(vd, orc.vp[layer]), f"step {step} layer {layer}: V pool"
            rel, mx = helpers.check_attention(layers[i]["out"].cpu().numpy(), outs_o[layer],
                                              zero_rows=[3],
                                              label=f"decode_step fused={fused} step {step}")
    say(f"decode_step fused={fused} p{partition_tokens}: 3 steps x 3 layers match the oracle")


@pytest.mark.parametrize("partition_tokens", [0, 16])
def test_fused_append_every_bf16_value(kv, partition_tokens):
    """64 requests x 8 KV heads x 128 dims = every bf16 pattern once as the
    new K (and, reversed, as the new V) of one fused launch, under 212 scales:
    the stored codes equal the oracle's. partition_tokens 0 runs the shared
    kernel (one partition each), 16 the persistent one (many partitions)."""
    batch, hkv, hq = 64, 8, 64
    lens = (np.arange(batch) * 7 % 97 + 1).astype(np.int32)     # 1 .. 97 tokens
    need = -(-lens // P)
    rng = np.random.default_rng(65536)
    num_pages = int(need.sum()) + 8
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((batch, int(need.max())), -1, np.int32)
    off = 0
    for b in range(batch):
        bt[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    if partition_tokens:
        from tests import wave_split_model as ws
        assert ws.uses_wave_kernel(batch, hkv, int(lens.max()), partition_tokens)
    vals = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(batch, hkv, 128)
    vvals = vals[::-1].copy()
    kn = torch.from_numpy(vals.view(np.int16)).to(DEV)
    vn = torch.from_numpy(vvals.view(np.int16)).to(DEV)
    q = torch.from_numpy(synth._f32_to_bf16_bits(rng.normal(0, 1, (batch, hq, 128))
                                                 .astype(np.float32)).view(np.int16)).to(DEV)
    junk = rng.integers(0, 0x7E, (num_pages, hkv, 2048)).astype(np.uint8)
    btt = torch.from_numpy(bt).to(DEV)
    seq = torch.from_numpy(lens).to(DEV)
    msl = int(lens.max())
    n = kv.paged_decode_attn_workspace_bytes(batch, hq, hkv, msl, partition_tokens)
    wsb = torch.zeros(max(n, 256), dtype=torch.uint8, device=DEV)
    out = torch.empty((batch, hq, 128), dtype=torch.float32, device=DEV)
    t = lens - 1
    pages = bt[np.arange(batch), t // P]
    scales = _encode_scales()
    starts = list(range(0, len(scales) - hkv + 1, hkv))
    if starts[-1] + hkv < len(scales):
        starts.append(len(scales) - hkv)             # the last few scales, in a full launch
    say(f"fused encode p{partition_tokens}: {len(starts)} launches x 65536 patterns")
    for i in starts:
        ks = scales[i:i + hkv].copy()
        vs = scales[::-1][i:i + hkv].copy()
        kp = torch.from_numpy(junk).to(DEV)
        vp = torch.from_numpy(junk[::-1].copy()).to(DEV)
        kv.paged_decode_attn_append(q, kn, vn, kp, vp, torch.from_numpy(ks).to(DEV),
                                    torch.from_numpy(vs).to(DEV), btt, seq, msl, out, 0.0884,
                                    workspace=wsb, partition_tokens=partition_tokens)
        torch.cuda.synchronize()
        kl = helpers.tiles_to_logical(kp.cpu().numpy(), "k", "fp8")    # [page][g][16][128]
        vl = helpers.tiles_to_logical(vp.cpu().numpy(), "v", "fp8")
        kgot = kl[pages, :, t % P]                                        # [batch][g][128]
        vgot = vl[pages, :, t % P]
        kwant = e4m3.quantize(vals, ks[None, :, None])
        vwant = e4m3.quantize(vvals, vs[None, :, None])
        bad = np.argwhere(kgot != kwant)
        assert bad.size == 0, (f"K scales {ks}: {len(bad)} codes differ, first "
                               f"x=0x{int(vals[tuple(bad[0])]):04x} "
                               f"got 0x{int(kgot[tuple(bad[0])]):02x} "
                               f"want 0x{int(kwant[tuple(bad[0])]):02x}")
        assert np.array_equal(vgot, vwant), f"V scales {vs}"
        # nothing else in the pool moved
        kl0 = helpers.tiles_to_logical(junk, "k", "fp8").copy()
        kl0[pages, :, t % P] = kwant
        assert np.array_equal(kl, kl0)


def test_ingest_layer_on_a_side_stream(kv):
    """ingest_layer with stream= a non-current torch stream (its scratch amax
    zeroed on that stream) equals the same call on the current stream."""
    wl = synth.mixed_8req(max_steps=1)
    kr, start = prompt_rows(wl, 0, "k", DEV)
    vr, _ = prompt_rows(wl, 0, "v", DEV)
    lens0 = torch.from_numpy(wl.seq_lens0.astype(np.int32)).to(DEV)
    results = []
    for side in (False, True):
        st = DeviceState(wl, kv, cache="fp8", device=DEV, layers=[0], fill=False,
                         scales={0: (np.ones(8, np.float32), np.ones(8, np.float32))})
        ks = torch.full((8,), 7.0, dtype=torch.float32, device=DEV)
        vs = torch.full((8,), 7.0, dtype=torch.float32, device=DEV)
        amax = torch.full((2, 8), 1e30, dtype=torch.float32, device=DEV)   # stale contents
        torch.cuda.synchronize()
        if side:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            # keep the current stream busy so a zeroing enqueued there would land late
            busy = torch.empty(64 << 20, dtype=torch.uint8, device=DEV)
            for _ in range(20):
                busy.add_(1)
            kv.ingest_layer(kr, vr, start, lens0, st.block_table, st.k_pool[0], st.v_pool[0],
                            wl.max_seq_len, ks, vs, amax=amax, stream=s)
            s.synchronize()
        else:
            kv.ingest_layer(kr, vr, start, lens0, st.block_table, st.k_pool[0], st.v_pool[0],
                            wl.max_seq_len, ks, vs, amax=amax)
        torch.cuda.synchronize()
        results.append((ks.cpu().numpy(), vs.cpu().numpy(), st.k_pool[0].cpu().numpy(),
                        st.v_pool[0].cpu().numpy()))
    for a, b in zip(*results):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    assert np.all(results[0][0] < 1.0) and np.all(results[0][1] < 1.0)


@pytest.mark.parametrize("fused", [True, False])
def test_prepared_calls_while_lengths_grow(kv, fused):
    """Calls prepared once with the largest length the loop reaches; each
    step's lengths are one longer. Four steps equal the oracle's four steps."""
    wl = synth.mixed_8req(max_steps=4)
    st = DeviceState(wl, kv, device=DEV)
    orc = OracleRun(st)
    sm = sm_scale_for(wl)
    seq_buf = torch.empty_like(st.seq_lens(0))
    pos_buf = torch.empty_like(st.tok_pos(0))
    q0, kn0, vn0 = st.step_layer_inputs(0, 0)
    q, kn, vn = torch.empty_like(q0), torch.empty_like(kn0), torch.empty_like(vn0)
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=DEV)
    ws = workspace(wl, 0)
    calls = [kv.kv_verify_tags(st.pool_tags, st.block_table, st.expected_tags, seq_buf,
                               st.abort, prepare=True)]
    if fused:
        calls.append(kv.paged_decode_attn_append(q, kn, vn, st.k_pool[0], st.v_pool[0],
                                                 st.k_scale[0], st.v_scale[0], st.block_table,
                                                 seq_buf, wl.max_seq_len, out, sm, workspace=ws,
                                                 abort=st.abort, prepare=True))
    else:
        calls.append(kv.kv_append_quant(kn, vn, st.tok_seq, pos_buf, st.block_table,
                                        st.k_scale[0], st.v_scale[0], st.k_pool[0],
                                        st.v_pool[0], abort=st.abort, prepare=True))
        calls.append(kv.paged_decode_attn(q, st.k_pool[0], st.v_pool[0], st.k_scale[0],
                                          st.v_scale[0], st.block_table, seq_buf,
                                          wl.max_seq_len, out, sm, workspace=ws,
                                          abort=st.abort, prepare=True))
    for step in range(4):
        seq_buf.copy_(st.seq_lens(step))
        pos_buf.copy_(st.tok_pos(step))
        sq, skn, svn = st.step_layer_inputs(0, step)
        q.copy_(sq)
        kn.copy_(skn)
        vn.copy_(svn)
        out.fill_(float("nan"))
        for c in calls:
            c()
        torch.cuda.synchronize()
        inputs = {0: (sq.view(torch.int16).cpu().numpy().view(np.uint16),
                      skn.cpu().numpy().view(np.uint16), svn.cpu().numpy().view(np.uint16))}
        ab_o, outs_o = orc.step(step, inputs)
        assert np.array_equal(st.abort.cpu().numpy(), ab_o)
        kd, vd = device_pool_logical(st, 0)
        assert np.array_equal(kd, orc.kp[0]) and np.array_equal(vd, orc.vp[0])
        helpers.check_attention(out.cpu().numpy(), outs_o[0], zero_rows=np.flatnonzero(ab_o),
                                label=f"prepared growing step {step}")
    say(f"prepared (fused={fused}): 4 growing steps match the oracle")
