"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: E4M3 codes and abort masks bit-exact; attention within rel-L2 <= 1e-3
and max |err| <= 5e-3 on identical dequantized inputs (the pools are checked
bit-exact first); aborted / empty / unmapped requests exactly zero.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import e4m3, paged
from synth.device import DeviceState
from tests import helpers
from tests.gpu_harness import (DEV, OracleRun, device_pool_logical, gpu_step, oracle_request,
                               say, sm_scale_for, workspace)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kv():
    import fp8_e4m3_paged_amd as k
    k.load()            # fails loudly if the library was not built
    return k


# ---------------------------------------------------------------------------
# exhaustive encode: every bf16 bit pattern through the bulk append
# ---------------------------------------------------------------------------
def _encode_scales():
    """Powers of two, random fp32 scales, and fp32(amax / 448) for bf16 amax
    values: the last kind puts many exact quotients a hair off an E4M3
    midpoint, where rounding the fp32 quotient alone would go wrong."""
    rng = np.random.default_rng(2024)
    fixed = [1.0, 0.5, 2.0, 8.0, 2.0 ** -7, 2.0 ** -20, 2.0 ** 20, 448.0 / 448.0]
    rnd = np.exp(rng.uniform(np.log(1e-4), np.log(30.0), 100))
    allv = e4m3.bf16_bits_to_f64(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    cand = np.unique(np.abs(allv[np.isfinite(allv) & (np.abs(allv) > 1e-3) & (np.abs(allv) < 1e3)]))
    amax = rng.choice(cand, size=100, replace=False).astype(np.float32) / np.float32(448)
    tiny = [float(np.float32(a) / np.float32(448)) for a in (4.0625, 2.15625, 4.3125, 2.1875)]
    return np.array(fixed + list(rnd) + list(amax) + tiny, dtype=np.float32)


def test_append_quant_every_bf16_value_many_scales(kv):
    hkv, ntok = 4, 128                     # 128 tokens x 4 heads x 128 dims = 65536 values
    say("exhaustive encode: 212 scales x 65536 bf16 patterns, K and V")
    vals = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(ntok, hkv, 128)
    vvals = vals[::-1].copy()
    bt = torch.arange(8, dtype=torch.int32, device=DEV).view(1, 8)
    seq = torch.zeros(ntok, dtype=torch.int32, device=DEV)
    pos = torch.arange(ntok, dtype=torch.int32, device=DEV)
    kn = torch.from_numpy(vals.view(np.int16)).to(DEV)
    vn = torch.from_numpy(vvals.view(np.int16)).to(DEV)
    scales = _encode_scales()
    assert len(scales) % hkv == 0
    for i in range(0, len(scales), hkv):
        ks = scales[i:i + hkv]
        vs = scales[::-1][i:i + hkv]
        kp = torch.zeros((8, hkv, 2048), dtype=torch.uint8, device=DEV)
        vp = torch.zeros((8, hkv, 2048), dtype=torch.uint8, device=DEV)
        kv.kv_append_quant(kn, vn, seq, pos, bt, torch.from_numpy(ks).to(DEV),
                           torch.from_numpy(vs.copy()).to(DEV), kp, vp)
        torch.cuda.synchronize()
        klog = helpers.tiles_to_logical(kp.cpu().numpy(), "k", "fp8")     # [page][g][16][128]
        vlog = helpers.tiles_to_logical(vp.cpu().numpy(), "v", "fp8")
        kgot = klog.transpose(0, 2, 1, 3).reshape(ntok, hkv, 128)
        vgot = vlog.transpose(0, 2, 1, 3).reshape(ntok, hkv, 128)
        kwant = e4m3.quantize(vals, ks[None, :, None])
        vwant = e4m3.quantize(vvals, vs[None, :, None])
        bad = np.argwhere(kgot != kwant)
        assert bad.size == 0, (f"K scale set {ks}: {len(bad)} codes differ, first "
                               f"x=0x{int(vals[tuple(bad[0])]):04x} got 0x{int(kgot[tuple(bad[0])]):02x}"
                               f" want 0x{int(kwant[tuple(bad[0])]):02x}")
        assert np.array_equal(vgot, vwant), f"V scale set {vs}"


def test_append_bf16_is_a_copy(kv):
    hkv, ntok = 4, 128
    vals = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(ntok, hkv, 128)
    bt = torch.arange(8, dtype=torch.int32, device=DEV).view(1, 8)
    seq = torch.zeros(ntok, dtype=torch.int32, device=DEV)
    pos = torch.arange(ntok, dtype=torch.int32, device=DEV)
    kn = torch.from_numpy(vals.view(np.int16)).to(DEV)
    kp = torch.zeros((8, hkv, 2048), dtype=torch.int16, device=DEV)
    vp = torch.zeros((8, hkv, 2048), dtype=torch.int16, device=DEV)
    kv.kv_append_bf16(kn, kn, seq, pos, bt, kp, vp)
    torch.cuda.synchronize()
    for pool, kind in ((kp, "k"), (vp, "v")):
        lg = helpers.tiles_to_logical(pool.cpu().numpy().view(np.uint16), kind, "bf16")
        assert np.array_equal(lg.transpose(0, 2, 1, 3).reshape(ntok, hkv, 128), vals)


# ---------------------------------------------------------------------------
# whole decode steps on the small configurations, everything compared
# ---------------------------------------------------------------------------
def _full_step_check(kv, wl, cache="fp8", partition_tokens=0, label="", fused=False):
    say(f"{label}: build device state ({wl.name}, {cache})")
    st = DeviceState(wl, kv, cache=cache, device=DEV)
    orc = OracleRun(st)
    for layer in st.layers:
        kd, vd = device_pool_logical(st, layer)
        assert np.array_equal(kd, orc.kp[layer]), f"{label}: K pool after fill, layer {layer}"
        assert np.array_equal(vd, orc.vp[layer]), f"{label}: V pool after fill, layer {layer}"
    say(f"{label}: step 0")
    ab, outs, inputs = gpu_step(st, 0, partition_tokens=partition_tokens, fused=fused)
    ab_o, outs_o = orc.step(0, inputs)
    assert np.array_equal(ab, ab_o), f"{label}: abort {ab} vs oracle {ab_o}"
    for layer in st.layers:
        kd, vd = device_pool_logical(st, layer)
        assert np.array_equal(kd, orc.kp[layer]), f"{label}: K pool after append"
        assert np.array_equal(vd, orc.vp[layer]), f"{label}: V pool after append"
        rel, mx = helpers.check_attention(outs[layer], outs_o[layer],
                                          zero_rows=np.flatnonzero(ab), label=label)
        say(f"{label}: layer {layer} rel_l2={rel:.2e} max_abs={mx:.2e}")
    return st, orc, ab


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_tiny_1req_step(kv, cache):
    st, _, ab = _full_step_check(kv, synth.tiny_1req(), cache, label=f"tiny/{cache}")
    assert not ab.any()


@pytest.mark.parametrize("partition_tokens", [0, 512])
def test_mixed_8req_step_with_stale_tag(kv, partition_tokens):
    wl = synth.mixed_8req()
    _, _, ab = _full_step_check(kv, wl, "fp8", partition_tokens, label=f"mixed8/p{partition_tokens}")
    assert np.flatnonzero(ab).tolist() == list(wl.stale)


def test_mixed_8req_bf16_step(kv):
    wl = synth.mixed_8req()
    _, _, ab = _full_step_check(kv, wl, "bf16", 1024, label="mixed8/bf16")
    assert np.flatnonzero(ab).tolist() == list(wl.stale)


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_tiny_1req_fused_append_attention_step(kv, cache):
    st, _, ab = _full_step_check(kv, synth.tiny_1req(), cache, label=f"tiny fused/{cache}",
                                 fused=True)
    assert not ab.any()


@pytest.mark.parametrize("partition_tokens", [0, 512, 4096])
def test_mixed_8req_fused_step_with_stale_tag(kv, partition_tokens):
    wl = synth.mixed_8req()
    _, _, ab = _full_step_check(kv, wl, "fp8", partition_tokens,
                                label=f"mixed8 fused/p{partition_tokens}", fused=True)
    assert np.flatnonzero(ab).tolist() == list(wl.stale)


def test_fused_equals_separate_calls_bit_for_bit(kv):
    wl = synth.mixed_8req(max_steps=3)
    a = DeviceState(wl, kv, device=DEV)
    b = DeviceState(wl, kv, device=DEV)
    for step in range(3):
        ab1, o1, _ = gpu_step(a, step, partition_tokens=1024, fused=False)
        ab2, o2, _ = gpu_step(b, step, partition_tokens=1024, fused=True)
        assert np.array_equal(ab1, ab2)
        assert np.array_equal(o1[0], o2[0], equal_nan=True)
        assert torch.equal(a.k_pool[0], b.k_pool[0]) and torch.equal(a.v_pool[0], b.v_pool[0])


@pytest.mark.parametrize("partition_tokens", [0, 512])
def test_step_captured_in_a_graph_replays_like_eager(kv, partition_tokens):
    """The tag check and the fused append + attention of one layer, captured
    in a HIP graph (through torch's graph capture on its capture stream) and
    replayed several times with eager work and synchronisations between
    replays: every replay equals the eager run bit for bit. (Replaying the
    same step rewrites the same codes into the same slot.)"""
    wl = synth.mixed_8req(max_steps=1)
    st = DeviceState(wl, kv, device=DEV, layers=[0])
    seq = st.seq_lens(0)
    q, kn, vn = st.step_layer_inputs(0, 0)
    ws = workspace(wl, partition_tokens)
    sm = sm_scale_for(wl)
    shape = (wl.batch, wl.num_q_heads, wl.head_dim)

    def step(out, abort):
        kv.kv_verify_tags(st.pool_tags, st.block_table, st.expected_tags, seq, abort)
        kv.paged_decode_attn_append(q, kn, vn, st.k_pool[0], st.v_pool[0], st.k_scale[0],
                                    st.v_scale[0], st.block_table, seq, wl.max_seq_len, out, sm,
                                    workspace=ws, abort=abort, partition_tokens=partition_tokens)

    out_e = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
    abort_e = torch.zeros(wl.batch, dtype=torch.uint8, device=DEV)
    step(out_e, abort_e)
    torch.cuda.synchronize()
    kp_e, vp_e = st.k_pool[0].clone(), st.v_pool[0].clone()
    assert int(abort_e.sum()) == 1

    out_g = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
    abort_g = torch.zeros(wl.batch, dtype=torch.uint8, device=DEV)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(out_g, abort_g)
    torch.cuda.synchronize()
    for r in range(4):
        out_g.fill_(float("nan"))
        abort_g.fill_(7)
        out_e.add_(0.0)                      # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(abort_g, abort_e), f"replay {r}: abort mask"
        assert torch.equal(out_g, out_e), f"replay {r}: attention output"
        assert torch.equal(st.k_pool[0], kp_e) and torch.equal(st.v_pool[0], vp_e)
    say(f"graph replay, partition {partition_tokens}: 4 replays equal the eager step")


# ---------------------------------------------------------------------------
# invariants on the GPU
# ---------------------------------------------------------------------------
def _attn(kv, st, layer, step, partition_tokens=0, sm=None, block_table=None, k_pool=None,
          v_pool=None, abort=None, max_seq_len=None):
    wl = st.wl
    q, _, _ = st.step_layer_inputs(layer, step)
    msl = max_seq_len or wl.max_seq_len
    out = torch.full((wl.batch, wl.num_q_heads, wl.head_dim), float("nan"), device=DEV)
    kv.paged_decode_attn(q, st.k_pool[layer] if k_pool is None else k_pool,
                         st.v_pool[layer] if v_pool is None else v_pool, st.k_scale[layer],
                         st.v_scale[layer], st.block_table if block_table is None else block_table,
                         st.seq_lens(step) - 1, msl, out,
                         sm_scale_for(wl) if sm is None else sm,
                         workspace=workspace(wl, partition_tokens, msl), abort=abort,
                         partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    return out.cpu().numpy(), q


def test_partition_size_independence_and_page_permutation(kv):
    wl = synth.mixed_8req()
    st = DeviceState(wl, kv, device=DEV)
    base, _ = _attn(kv, st, 0, 0, partition_tokens=16384)
    for pt in (16, 32, 48, 512, 1024, 4096, 0):
        out, _ = _attn(kv, st, 0, 0, partition_tokens=pt)
        helpers.check_attention(out, base, label=f"partition {pt} vs one partition")
    # move every physical page to a new place: the output must not change at all
    perm = np.random.default_rng(5).permutation(wl.num_pages)
    inv = torch.from_numpy(np.argsort(perm).astype(np.int32)).to(DEV)
    permt = torch.from_numpy(perm.astype(np.int64)).to(DEV)
    kp2 = st.k_pool[0][permt].contiguous()
    vp2 = st.v_pool[0][permt].contiguous()
    bt2 = st.block_table.clone()
    m = (bt2 >= 0) & (bt2 < wl.num_pages)
    bt2[m] = inv[bt2[m].long()]
    for pt in (0, 512):
        a, _ = _attn(kv, st, 0, 0, partition_tokens=pt)
        b, _ = _attn(kv, st, 0, 0, partition_tokens=pt, block_table=bt2, k_pool=kp2, v_pool=vp2)
        assert np.array_equal(a, b)


@pytest.mark.parametrize("partition_tokens", [1024, 64])
def test_zero_temperature_is_mean_of_v(kv, partition_tokens):
    """sm_scale = 0: every score is 0 and the output is the plain mean of V.
    1,024-token partitions run the shared kernel, 64-token ones (8 requests x 8
    KV heads x up to 128 partitions) the persistent one."""
    wl = synth.mixed_8req()
    st = DeviceState(wl, kv, device=DEV)
    out, _ = _attn(kv, st, 0, 0, sm=0.0, partition_tokens=partition_tokens)
    vlog = device_pool_logical(st, 0)[1]
    for b in range(wl.batch):
        L = int(wl.seq_lens0[b])
        V = paged.dequant_request(vlog, wl.block_table[b], L, 16, st.v_scale_host[0], "fp8")
        want = np.repeat(V.mean(axis=1), wl.num_q_heads // wl.num_kv_heads, axis=0)
        helpers.check_attention(out[b:b + 1], want[None], label=f"mean V, request {b}")


# ---------------------------------------------------------------------------
# edge cases on a hand-made state
# ---------------------------------------------------------------------------
def _edge_state(kv, cache, hq, hkv, lens, pool_pages=40, nan_fill=True):
    """Pool pages pre-filled with stale bytes (NaN codes included) before the
    requests' tokens are appended, so unwritten slots hold garbage."""
    rng = np.random.default_rng(99)
    batch = len(lens)
    need = [max(1, -(-L // 16)) for L in lens]
    perm = rng.permutation(pool_pages).astype(np.int32)
    bt = np.full((batch, max(need) + 1), -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        bt[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    dt = torch.uint8 if cache == "fp8" else torch.int16
    if cache == "fp8":
        junk = rng.integers(0, 256, (pool_pages, hkv, 2048)).astype(np.uint8)
        if nan_fill:
            junk[:, :, ::7] = 0x7F
        kp = torch.from_numpy(junk).to(DEV)
        vp = torch.from_numpy(junk[::-1].copy()).to(DEV)
    else:
        junk = rng.integers(0, 65536, (pool_pages, hkv, 2048)).astype(np.uint16)
        if nan_fill:
            junk[:, :, ::7] = 0x7FC0
        kp = torch.from_numpy(junk.view(np.int16)).to(DEV)
        vp = torch.from_numpy(junk[::-1].copy().view(np.int16)).to(DEV)
    assert kp.dtype == dt
    # append real tokens for every position < L
    seqs = np.concatenate([np.full(L, b, np.int32) for b, L in enumerate(lens)] + [np.zeros(0, np.int32)])
    poss = np.concatenate([np.arange(L, dtype=np.int32) for L in lens] + [np.zeros(0, np.int32)])
    kvals = synth._f32_to_bf16_bits(rng.normal(0, 1, (len(seqs), hkv, 128)).astype(np.float32))
    vvals = synth._f32_to_bf16_bits(rng.normal(0, 0.5, (len(seqs), hkv, 128)).astype(np.float32))
    ks = np.full(hkv, 4.3 / 448, dtype=np.float32) * (1 + np.arange(hkv, dtype=np.float32) / 8)
    vs = np.full(hkv, 2.2 / 448, dtype=np.float32)
    btt = torch.from_numpy(bt).to(DEV)
    kst, vst = torch.from_numpy(ks).to(DEV), torch.from_numpy(vs).to(DEV)
    if len(seqs):
        args = (torch.from_numpy(kvals.view(np.int16)).to(DEV),
                torch.from_numpy(vvals.view(np.int16)).to(DEV),
                torch.from_numpy(seqs).to(DEV), torch.from_numpy(poss).to(DEV), btt)
        if cache == "fp8":
            kv.kv_append_quant(*args, kst, vst, kp, vp)
        else:
            kv.kv_append_bf16(*args, kp, vp)
    q = synth._f32_to_bf16_bits(rng.normal(0, 1, (batch, hq, 128)).astype(np.float32))
    torch.cuda.synchronize()
    return dict(bt=bt, btt=btt, kp=kp, vp=vp, ks=ks, vs=vs, kst=kst, vst=vst, q=q,
                lens=np.array(lens, np.int32))


def _edge_run(kv, e, cache, lens=None, abort=None, max_seq_len=None, partition_tokens=0,
              bt=None):
    lens = e["lens"] if lens is None else np.asarray(lens, np.int32)
    batch, hq, _ = e["q"].shape
    msl = int(lens.max()) if max_seq_len is None else max_seq_len
    out = torch.full((batch, hq, 128), float("nan"), device=DEV)
    n = kv.paged_decode_attn_workspace_bytes(
        batch, hq, e["kp"].shape[1], msl, partition_tokens,
        cache_dtype=kv.KV_CACHE_FP8_E4M3 if cache == "fp8" else kv.KV_CACHE_BF16)
    ws = torch.zeros(max(n, 256), dtype=torch.uint8, device=DEV)
    btt = e["btt"] if bt is None else torch.from_numpy(bt).to(DEV)
    kv.paged_decode_attn(torch.from_numpy(e["q"].view(np.int16)).to(DEV), e["kp"], e["vp"],
                         e["kst"] if cache == "fp8" else None,
                         e["vst"] if cache == "fp8" else None, btt,
                         torch.from_numpy(lens).to(DEV), msl, out, 0.0883883,
                         workspace=ws,
                         abort=None if abort is None else torch.from_numpy(
                             np.asarray(abort, np.uint8)).to(DEV),
                         partition_tokens=partition_tokens,
                         cache_dtype=0 if cache == "fp8" else 1)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _edge_oracle(e, cache, lens, abort=None, bt=None):
    kt = e["kp"].cpu().numpy()
    vt = e["vp"].cpu().numpy()
    if cache == "bf16":
        kt, vt = kt.view(np.uint16), vt.view(np.uint16)
    kl = helpers.tiles_to_logical(kt, "k", cache)
    vl = helpers.tiles_to_logical(vt, "v", cache)
    return paged.decode_attn(e["q"], kl, vl, e["ks"], e["vs"], e["bt"] if bt is None else bt,
                             np.asarray(lens, np.int32), 0.0883883, cache, abort)


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
@pytest.mark.parametrize("hq,hkv", [(8, 1), (16, 2), (4, 4), (32, 2), (4, 2), (6, 2), (12, 3),
                                     (24, 4), (24, 2), (10, 2), (14, 1), (7, 1), (18, 2),
                                     (20, 2), (11, 1), (26, 2), (15, 1)])
def test_edge_lengths_groups_and_garbage_slots(kv, cache, hq, hkv):
    """Every GQA group size from 1 to 16 (G = hq / hkv), lengths around page and
    page-pair edges, an empty request, and slots past each length holding
    garbage, at the automatic and three short partition sizes."""
    lens = [1, 2, 15, 16, 17, 31, 33, 100, 0, 47]
    e = _edge_state(kv, cache, hq, hkv, lens)
    for pt in (0, 16, 32, 64):
        got = _edge_run(kv, e, cache, partition_tokens=pt)
        want = _edge_oracle(e, cache, lens)
        helpers.check_attention(got, want, zero_rows=[8], label=f"edge {cache} G={hq//hkv} p{pt}")
        # one token: exactly V0 (dequantized), the first check of the decode path
        assert np.allclose(got[0], want[0], rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (12, 4), (20, 4), (32, 2)])
@pytest.mark.parametrize("pt", [0, 32])
def test_fused_append_equals_separate_calls_any_group(kv, cache, hq, hkv, pt):
    """The fused append + attention call against kv_append_* followed by
    paged_decode_attn on a twin state, at group sizes 1, 3, 5 and 16 and two
    partition sizes: outputs and pools bit for bit, and the output within the
    oracle's tolerance. The new tokens land first in a page, last in a page,
    mid-page and in requests that had none."""
    lens = [1, 2, 15, 16, 17, 31, 33, 100, 0, 47]          # tokens before the step
    plus = [L + 1 for L in lens]                              # after it
    a = _edge_state(kv, cache, hq, hkv, plus)
    b = _edge_state(kv, cache, hq, hkv, plus)
    rng = np.random.default_rng(5)
    batch = len(lens)
    kb = synth._f32_to_bf16_bits(rng.normal(0, 1, (batch, hkv, 128)).astype(np.float32))
    vb = synth._f32_to_bf16_bits(rng.normal(0, 0.5, (batch, hkv, 128)).astype(np.float32))
    kn = torch.from_numpy(kb.view(np.int16)).to(DEV)
    vn = torch.from_numpy(vb.view(np.int16)).to(DEV)
    seq = torch.from_numpy(np.array(plus, np.int32)).to(DEV)
    msl = max(plus)
    q = torch.from_numpy(a["q"].view(np.int16)).to(DEV)
    fp8 = cache == "fp8"
    cd = kv.KV_CACHE_FP8_E4M3 if fp8 else kv.KV_CACHE_BF16
    n = kv.paged_decode_attn_workspace_bytes(batch, hq, hkv, msl, pt, cache_dtype=cd)
    ws_a = torch.zeros(max(n, 256), dtype=torch.uint8, device=DEV)
    ws_b = torch.zeros(max(n, 256), dtype=torch.uint8, device=DEV)
    out_f = torch.full((batch, hq, 128), float("nan"), device=DEV)
    out_s = torch.full((batch, hq, 128), float("nan"), device=DEV)
    sm = 0.0883883
    kv.paged_decode_attn_append(q, kn, vn, a["kp"], a["vp"], a["kst"] if fp8 else None,
                                a["vst"] if fp8 else None, a["btt"], seq, msl, out_f, sm,
                                workspace=ws_a, partition_tokens=pt, cache_dtype=cd)
    tok_seq = torch.arange(batch, dtype=torch.int32, device=DEV)
    tok_pos = seq - 1
    if fp8:
        kv.kv_append_quant(kn, vn, tok_seq, tok_pos, b["btt"], b["kst"], b["vst"], b["kp"],
                           b["vp"])
    else:
        kv.kv_append_bf16(kn, vn, tok_seq, tok_pos, b["btt"], b["kp"], b["vp"])
    kv.paged_decode_attn(q, b["kp"], b["vp"], b["kst"] if fp8 else None,
                         b["vst"] if fp8 else None, b["btt"], seq, msl, out_s, sm,
                         workspace=ws_b, partition_tokens=pt, cache_dtype=cd)
    torch.cuda.synchronize()
    assert torch.equal(out_f, out_s), "fused output differs from the separate calls"
    assert torch.equal(a["kp"], b["kp"]) and torch.equal(a["vp"], b["vp"])
    want = _edge_oracle(b, cache, plus)
    helpers.check_attention(out_f.cpu().numpy(), want, label=f"fused {cache} G={hq // hkv} p{pt}")


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_edge_abort_bad_ids_and_overlong(kv, cache):
    lens = [20, 40, 5, 64, 16]
    e = _edge_state(kv, cache, 8, 1, lens)
    bt = e["bt"].copy()
    bt[1, 1] = 10 ** 6          # request 1 reads an out-of-pool page
    bt[3, 0] = -5               # request 3 too
    abort = [0, 0, 1, 0, 0]     # request 2 aborted by the tag check
    for pt in (0, 16):
        got = _edge_run(kv, e, cache, abort=abort, partition_tokens=pt, bt=bt)
        want = _edge_oracle(e, cache, lens, abort=np.array(abort, np.uint8), bt=bt)
        helpers.check_attention(got, want, zero_rows=[1, 2, 3], label=f"abort/bad {cache} p{pt}")
    # a length above max_seq_len, or beyond the table row, is refused (zeros)
    got = _edge_run(kv, e, cache, lens=[20, 40, 5, 64, 16], max_seq_len=39)
    assert np.all(got[1] == 0) and np.all(got[3] == 0) and np.any(got[0] != 0)
    got = _edge_run(kv, e, cache, lens=[20, 40, 5, 16 * e["bt"].shape[1] + 1, 16])
    assert np.all(got[3] == 0)


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_automatic_split_of_one_long_request(kv, cache):
    """A request of 9,193 tokens and one of 17 pages, 64 query / 8 KV heads,
    automatic partitions: FP8 gets 12 of 768 tokens and BF16 16 of 576 (at
    least 192 KiB of K and V per partition), which the reduction combines in
    one round trip (rows of up to 16 slots). Every row against the oracle, and
    again with explicit 512-token partitions (18 slots: the two-pass path)."""
    lens = [9193, 17 * 16]
    need = sum(max(1, -(-L // 16)) for L in lens)
    e = _edge_state(kv, cache, 64, 8, lens, pool_pages=need + 8)
    cd = kv.KV_CACHE_FP8_E4M3 if cache == "fp8" else kv.KV_CACHE_BF16
    pt = kv.paged_decode_attn_partition_tokens(len(lens), 8, max(lens), 0, cd)
    assert pt == (768 if cache == "fp8" else 576)
    assert -(-max(lens) // pt) <= 16
    want = _edge_oracle(e, cache, lens)
    got = _edge_run(kv, e, cache)
    helpers.check_attention(got, want, label=f"automatic split {cache}")
    got512 = _edge_run(kv, e, cache, partition_tokens=512)
    helpers.check_attention(got512, want, label=f"512-token partitions {cache}")


def _uses_persistent_kernel(batch, hkv, max_len, pt):
    """Whether the library picks its persistent kernel
    (short partitions and enough of them to give every CU a 4-wave group)."""
    parts = -(-max_len // pt)
    return parts > 1 and pt <= 2048 and batch <= 4096 and batch * hkv * parts >= 1024


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
@pytest.mark.parametrize("hq", [8, 16, 24, 32, 40, 48, 56, 64, 72, 80, 88, 96, 104, 112, 120,
                                128])
def test_wave_mode_edges_aborts_and_bad_ids(kv, cache, hq):
    """Every GQA group size from 1 to 16 (8 KV heads). A batch large enough for
    the persistent kernel, with ragged
    lengths (1 token, page and partition boundaries, empty requests) and
    aborted and badly mapped requests between valid ones, so the kernel's
    per-request numbering of its work items has to skip them."""
    hkv = 8
    base = [1, 2, 15, 16, 17, 31, 33, 100, 0, 47, 64, 65, 129, 200]
    lens = base * 10
    need = sum(max(1, -(-L // 16)) for L in lens)
    e = _edge_state(kv, cache, hq, hkv, lens, pool_pages=need + 16)
    bt = e["bt"].copy()
    bt[5, 1] = 10 ** 6          # L = 31: its second page is outside the pool
    bt[60, 1] = -2              # L = 17: likewise
    bt[12, 8] = 10 ** 6         # L = 129: only the last (one-token) page is bad
    abort = np.zeros(len(lens), np.uint8)
    abort[4::9] = 1
    zero = sorted({b for b, L in enumerate(lens) if L == 0} | {5, 60, 12} |
                  set(np.flatnonzero(abort).tolist()))
    want = _edge_oracle(e, cache, lens, abort=abort, bt=bt)
    for pt in (16, 32, 48, 64, 80):            # 1 to 5 pages per partition, odd ones too
        assert _uses_persistent_kernel(len(lens), hkv, max(lens), pt)
        got = _edge_run(kv, e, cache, abort=abort, partition_tokens=pt, bt=bt)
        helpers.check_attention(got, want, zero_rows=zero,
                                label=f"wave mode {cache} G={hq // hkv} p{pt}")
        b1 = lens.index(1)
        assert np.allclose(got[b1], want[b1], rtol=2e-6, atol=1e-7)


def test_verify_tags_cases(kv):
    rng = np.random.default_rng(17)
    num_pages, batch, width = 300, 9, 40
    tags = rng.integers(0, 2 ** 32, num_pages, dtype=np.uint64).astype(np.uint32)
    bt = rng.integers(0, num_pages, (batch, width)).astype(np.int32)
    exp = tags[bt].copy()
    lens = np.array([0, 1, 16, 17, 640, 641, -3, 300, 200], np.int32)
    bt[2, 1] = -1                      # past request 2's pages: ignored
    bt[3, 1] = -1                      # request 3 reads it: abort
    exp[4, 39] ^= 1                    # last page of request 4: abort
    exp[7, 19] ^= 1 << 31              # request 7 (300 tokens = 19 pages): page 19 not read
    exp[8, 12] ^= 1                    # request 8: abort
    assert paged.verify_tags(tags, bt, exp, lens, 16).tolist() == [0, 0, 0, 1, 1, 1, 1, 0, 1]
    cases = [lens, np.full(batch, 0, np.int32), np.full(batch, 640, np.int32)]
    for ls in cases:
        want = paged.verify_tags(tags, bt, exp, ls, 16)
        ab = torch.full((batch,), 7, dtype=torch.uint8, device=DEV)
        kv.kv_verify_tags(torch.from_numpy(tags.view(np.int32)).to(DEV),
                          torch.from_numpy(bt).to(DEV),
                          torch.from_numpy(exp.view(np.int32)).to(DEV),
                          torch.from_numpy(ls).to(DEV), ab)
        torch.cuda.synchronize()
        assert np.array_equal(ab.cpu().numpy(), want), (ls, ab.cpu().numpy(), want)


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_maximum_partition_count(kv, cache):
    """131,072 tokens in 16-token partitions: 8,192 partitions, the most the
    library accepts, in the persistent kernel. The reduce then combines 8,193
    slots of the long request's rows, a few hundred of them non-empty, four
    wavefronts per row; the short request and an empty one share the launch."""
    lens = [131_072, 5_000, 0]
    need = sum(max(1, -(-L // 16)) for L in lens)
    e = _edge_state(kv, cache, 8, 1, lens, pool_pages=need + 4)
    assert _uses_persistent_kernel(len(lens), 1, max(lens), 16)
    got = _edge_run(kv, e, cache, partition_tokens=16)
    want = _edge_oracle(e, cache, lens)
    helpers.check_attention(got, want, zero_rows=[2], label=f"8192 partitions {cache}")
    # an invalid page id deep inside the long request, and the short one aborted:
    # both rows zero, seen by whichever wavefront of the reduction holds the slot
    bt = e["bt"].copy()
    bt[0, 6_000] = -1
    got = _edge_run(kv, e, cache, partition_tokens=16, bt=bt, abort=[0, 1, 0])
    assert np.all(got[0] == 0) and np.all(got[1] == 0) and np.all(got[2] == 0)


@pytest.mark.parametrize("split", [False, True])
def test_verify_tags_long_rows(kv, split):
    """Rows of up to 5,000 pages (80k tokens), more than one sweep of the
    whole-row workgroup's 1,024 threads, or (split) three 2,048-page chunks
    checked by three workgroups that combine through the counter workspace: a
    failing page anywhere (first, middle, last, either side of a chunk edge,
    the one page of a last sweep) aborts exactly its request, pages past a
    request's length are ignored, and flags that held 1 or junk before the
    call are overwritten with the oracle's 0 / 1. The counters are back at
    zero after every call."""
    rng = np.random.default_rng(23)
    num_pages, batch, width = 50_000, 12, 5_000
    tags = rng.integers(0, 2 ** 32, num_pages, dtype=np.uint64).astype(np.uint32)
    bt = rng.integers(0, num_pages, (batch, width)).astype(np.int32)
    exp = tags[bt].copy()
    lens = np.array([16 * 5_000, 16 * 5_000, 16 * 5_000, 16 * 4_097, 16 * 1_024 + 1, 0, -1,
                     16 * 5_000 + 1, 16 * 3_000, 16 * 2_048, 16 * 5_000, 16 * 1_500], np.int32)
    exp[0, 0] ^= 1                     # the first page
    exp[1, 2_500] ^= 1 << 7            # a middle one
    exp[2, 4_999] ^= 1 << 31           # the last page of a full row
    exp[3, 4_096] ^= 1                 # the one page of a 4,097-page request's last sweep
    bt[4, 1_024] = num_pages           # a page id just outside the pool
    bt[8, 3_000] = -1                  # past request 8's pages: ignored
    exp[9, 2_048] ^= 1                 # likewise
    exp[10, 2_047] ^= 1                # the last page of a first chunk
    bt[11, 1_499] = -7                 # last page of a 1500-page request
    want = paged.verify_tags(tags, bt, exp, lens, 16)
    assert want.tolist() == [1, 1, 1, 1, 1, 0, 1, 1, 0, 0, 1, 1]
    ws = None
    if split:
        n = kv.kv_verify_tags_workspace_bytes(batch, width)
        assert n == 8 * batch
        ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    for fill in (0, 1, 0xA5):
        ab = torch.full((batch,), fill, dtype=torch.uint8, device=DEV)
        kv.kv_verify_tags(torch.from_numpy(tags.view(np.int32)).to(DEV),
                          torch.from_numpy(bt).to(DEV),
                          torch.from_numpy(exp.view(np.int32)).to(DEV),
                          torch.from_numpy(lens).to(DEV), ab, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(ab.cpu().numpy(), want), (fill, ab.cpu().numpy(), want)
        if split:
            assert int(ws.count_nonzero()) == 0


def test_split_verify_captured_in_a_graph_replays_fresh(kv):
    """The split tag check (5,000-page rows over three workgroups per request,
    combining through the counter workspace) captured in a HIP graph and
    replayed with the expected tags changed between replays: every replay
    gives the oracle's mask for the tags it read, overwrites junk flags, and
    leaves the counters at zero for the next replay."""
    rng = np.random.default_rng(29)
    num_pages, batch, width = 40_000, 6, 5_000
    tags = rng.integers(0, 2 ** 32, num_pages, dtype=np.uint64).astype(np.uint32)
    bt = rng.integers(0, num_pages, (batch, width)).astype(np.int32)
    exp = tags[bt].copy()
    lens = np.array([16 * 5_000, 16 * 4_500, 16 * 3_000, 16 * 2_049, 16 * 5_000, 16 * 100],
                    np.int32)
    exp[1, 4_200] ^= 1                                       # request 1 fails throughout
    d_tags = torch.from_numpy(tags.view(np.int32)).to(DEV)
    d_bt = torch.from_numpy(bt).to(DEV)
    d_exp = torch.from_numpy(exp.view(np.int32)).to(DEV)
    d_lens = torch.from_numpy(lens).to(DEV)
    ws = torch.zeros(kv.kv_verify_tags_workspace_bytes(batch, width), dtype=torch.uint8,
                     device=DEV)
    ab = torch.zeros(batch, dtype=torch.uint8, device=DEV)
    kv.kv_verify_tags(d_tags, d_bt, d_exp, d_lens, ab, workspace=ws)   # warm-up, eager
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kv.kv_verify_tags(d_tags, d_bt, d_exp, d_lens, ab, workspace=ws)
    torch.cuda.synchronize()
    # per replay, one more page to flip: a chunk edge, a last page, an ignored page
    flips = [(0, 2_048), (4, 4_999), (3, 2_048), (5, 100), (2, 2_999)]
    for r, (b, pg) in enumerate(flips):
        cur = exp.copy()
        cur[b, pg] ^= 1 << (r + 3)
        d_exp.copy_(torch.from_numpy(cur.view(np.int32)))
        ab.fill_(0xA5 if r % 2 else 1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = paged.verify_tags(tags, bt, cur, lens, 16)
        assert np.array_equal(ab.cpu().numpy(), want), (r, ab.cpu().numpy(), want)
        assert int(ws.count_nonzero()) == 0, f"replay {r}: counters not reset"
    say("split tag check: 5 graph replays with changed tags match the oracle")


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_wave_mode_even_page_split_long_partitions(kv, cache):
    """Partitions of 256 to 2048 tokens in the wave-mode kernel, which splits
    the work evenly by pages: wavefronts start inside partitions, some inside a
    request's last partition. Every output against the oracle, then the fused
    append + attention against the separate calls, bit for bit, and again
    against the oracle on the pools the fused launch wrote."""
    hq, hkv = 64, 8
    rng = np.random.default_rng(7)
    lens = rng.integers(1, 3000, 72)
    lens[[3, 40]] = 0
    lens[[10, 11, 12, 13, 14]] = [2048, 2049, 4096, 1, 16]
    lens = lens.tolist()
    need = sum(max(1, -(-L // 16)) for L in lens)
    e = _edge_state(kv, cache, hq, hkv, lens, pool_pages=need + 8)
    zero = [b for b, L in enumerate(lens) if L == 0]
    want = _edge_oracle(e, cache, lens)
    for pt in (256, 1024, 2048):
        assert _uses_persistent_kernel(len(lens), hkv, max(lens), pt)
        got = _edge_run(kv, e, cache, partition_tokens=pt)
        helpers.check_attention(got, want, zero_rows=zero, label=f"page split {cache} p{pt}")

    # the fused path: a new row for position L - 1 of every non-empty request
    batch = len(lens)
    kn = synth._f32_to_bf16_bits(rng.normal(0, 1, (batch, hkv, 128)).astype(np.float32))
    vn = synth._f32_to_bf16_bits(rng.normal(0, 0.5, (batch, hkv, 128)).astype(np.float32))
    knt = torch.from_numpy(kn.view(np.int16)).to(DEV)
    vnt = torch.from_numpy(vn.view(np.int16)).to(DEV)
    live = np.array([b for b, L in enumerate(lens) if L > 0], np.int32)
    pos = np.array([lens[b] - 1 for b in live], np.int32)
    q = torch.from_numpy(e["q"].view(np.int16)).to(DEV)
    seq = torch.from_numpy(np.array(lens, np.int32)).to(DEV)
    msl = max(lens)
    for pt in (1024, 2048):
        n = kv.paged_decode_attn_workspace_bytes(batch, hq, hkv, msl, pt)
        ws = torch.zeros(max(n, 256), dtype=torch.uint8, device=DEV)
        kp_a, vp_a = e["kp"].clone(), e["vp"].clone()
        kp_b, vp_b = e["kp"].clone(), e["vp"].clone()
        li = torch.from_numpy(live).to(DEV)
        args = (knt[li], vnt[li], li, torch.from_numpy(pos).to(DEV), e["btt"])
        if cache == "fp8":
            kv.kv_append_quant(*args, e["kst"], e["vst"], kp_a, vp_a)
        else:
            kv.kv_append_bf16(*args, kp_a, vp_a)
        ks = e["kst"] if cache == "fp8" else None
        vs = e["vst"] if cache == "fp8" else None
        dt = 0 if cache == "fp8" else 1
        out_a = torch.full((batch, hq, 128), float("nan"), device=DEV)
        out_b = torch.full((batch, hq, 128), float("nan"), device=DEV)
        kv.paged_decode_attn(q, kp_a, vp_a, ks, vs, e["btt"], seq, msl, out_a, 0.0883883,
                             workspace=ws, partition_tokens=pt, cache_dtype=dt)
        kv.paged_decode_attn_append(q, knt, vnt, kp_b, vp_b, ks, vs, e["btt"], seq, msl, out_b,
                                    0.0883883, workspace=ws, partition_tokens=pt,
                                    cache_dtype=dt)
        torch.cuda.synchronize()
        assert torch.equal(kp_a, kp_b) and torch.equal(vp_a, vp_b), f"fused pools p{pt}"
        assert torch.equal(out_a, out_b), f"fused output p{pt}"
    e2 = dict(e, kp=kp_b, vp=vp_b)
    helpers.check_attention(out_b.cpu().numpy(), _edge_oracle(e2, cache, lens), zero_rows=zero,
                            label=f"page split fused {cache}")


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_large_batches_at_the_kernel_limits(kv, cache):
    """Thousands of short requests (GQA 8/1): 4,096, the largest batch the
    persistent kernel takes (its per-request prefix fills the most LDS), and
    4,097, one past it, where the shared kernel runs the same 16-token
    partitions and the reduce covers 32,776 rows; then 20,000 requests in one
    partition each. Ragged lengths from 1 to 96 tokens with empty and aborted
    requests scattered through; every row against the oracle."""
    hq, hkv = 8, 1
    rng = np.random.default_rng(4097)
    lens = rng.integers(1, 97, 4097)
    lens[::511] = 0
    lens = lens.tolist()
    need = sum(max(1, -(-L // 16)) for L in lens)
    e = _edge_state(kv, cache, hq, hkv, lens, pool_pages=need + 16)
    abort = np.zeros(len(lens), np.uint8)
    abort[7::613] = 1
    for batch in (4096, 4097):
        sub = dict(e, q=e["q"][:batch], bt=e["bt"][:batch], btt=e["btt"][:batch],
                   lens=e["lens"][:batch])
        ln = lens[:batch]
        ab = abort[:batch]
        assert _uses_persistent_kernel(batch, hkv, max(ln), 16) == (batch <= 4096)
        zero = sorted({b for b, L in enumerate(ln) if L == 0} | set(np.flatnonzero(ab).tolist()))
        want = _edge_oracle(sub, cache, ln, abort=ab)
        got = _edge_run(kv, sub, cache, abort=ab, partition_tokens=16)
        helpers.check_attention(got, want, zero_rows=zero, label=f"batch {batch} {cache} p16")
    if cache == "bf16":
        return
    # 20,000 requests, one partition each (the shared kernel's grid of 20,000
    # workgroups, no reduce), and the batched tag check over all of them
    big = 20_000
    lens2 = rng.integers(1, 49, big)
    lens2[::997] = 0
    lens2 = lens2.tolist()
    need2 = sum(max(1, -(-L // 16)) for L in lens2)
    e2 = _edge_state(kv, cache, hq, hkv, lens2, pool_pages=need2 + 16)
    zero2 = [b for b, L in enumerate(lens2) if L == 0]
    assert kv.paged_decode_attn_partition_tokens(big, hkv, max(lens2), 0) >= max(lens2)
    want2 = _edge_oracle(e2, cache, lens2)
    got2 = _edge_run(kv, e2, cache)
    helpers.check_attention(got2, want2, zero_rows=zero2, label=f"batch {big} {cache}")
    tags = rng.integers(0, 2 ** 32, need2 + 16, dtype=np.uint64).astype(np.uint32)
    bt2 = e2["bt"]
    exp = tags[np.clip(bt2, 0, None)]
    stale = rng.choice(big, 5, replace=False)
    for b in stale:
        if lens2[b] > 0:
            exp[b, 0] ^= 1
    want_ab = paged.verify_tags(tags, bt2, exp, np.array(lens2, np.int32), 16)
    ab = torch.full((big,), 0xA5, dtype=torch.uint8, device=DEV)
    kv.kv_verify_tags(torch.from_numpy(tags.view(np.int32)).to(DEV), e2["btt"],
                      torch.from_numpy(exp.view(np.int32)).to(DEV),
                      torch.from_numpy(np.array(lens2, np.int32)).to(DEV), ab)
    torch.cuda.synchronize()
    assert np.array_equal(ab.cpu().numpy(), want_ab)
    assert sorted(np.flatnonzero(want_ab).tolist()) == sorted(int(b) for b in stale if lens2[b] > 0)


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_pools_larger_than_4gib(kv, cache):
    """A 330,000-page pool (5.4 GB per K or V array with FP8 tiles, 10.8 GB
    with BF16) whose requests live in its top 30,000 pages, so every tile
    offset lies beyond 2^32 bytes (one request at the bottom for contrast):
    the prompts calibrated and ingested there, then one fused append +
    attention step in the shared kernel (automatic split) and in the
    persistent kernel (64-token partitions), after the tag check. Scales,
    every code of every request and every output against the oracle."""
    from oracle import ingest
    hq, hkv, num_pages = 64, 8, 330_000
    rng = np.random.default_rng(4242)
    lens = [1, 17, 1000, 4096, 9000, 20000]
    batch = len(lens)
    need = [-(-L // 16) for L in lens]
    top = rng.permutation(np.arange(num_pages - 30_000, num_pages))
    ids, off = [np.array([3])], 0
    for n in need[1:]:
        ids.append(top[off:off + n])
        off += n
    bt = np.full((batch, max(need)), -1, np.int32)
    for b in range(batch):
        bt[b, :need[b]] = ids[b]
    assert bt[1:].max() >= num_pages - 30_000 and (num_pages - 30_000) * hkv * 2048 > 2 ** 32
    prompt = [L - 1 for L in lens]                      # the last token comes with the step
    rows_k = synth._f32_to_bf16_bits(rng.normal(0, 1, (sum(prompt), hkv, 128)).astype(np.float32))
    rows_v = synth._f32_to_bf16_bits(rng.normal(0, 0.5, (sum(prompt), hkv, 128)).astype(np.float32))
    start = np.concatenate([[0], np.cumsum(prompt)[:-1]]).astype(np.int32)
    new_k = synth._f32_to_bf16_bits(rng.normal(0, 1, (batch, hkv, 128)).astype(np.float32))
    new_v = synth._f32_to_bf16_bits(rng.normal(0, 0.5, (batch, hkv, 128)).astype(np.float32))
    q = synth._f32_to_bf16_bits(rng.normal(0, 1, (batch, hq, 128)).astype(np.float32))
    fp8 = cache == "fp8"
    cd = kv.KV_CACHE_FP8_E4M3 if fp8 else kv.KV_CACHE_BF16
    dt = torch.uint8 if fp8 else torch.int16
    fill = 0x7F if fp8 else 0x7FC0                      # NaN everywhere no request writes
    btt = torch.from_numpy(bt).to(DEV)
    tags = rng.integers(0, 2 ** 32, num_pages, dtype=np.uint64).astype(np.uint32)
    exp = tags[np.clip(bt, 0, None)]
    d_tags = torch.from_numpy(tags.view(np.int32)).to(DEV)
    d_exp = torch.from_numpy(exp.view(np.int32)).to(DEV)
    d_lens = torch.from_numpy(np.array(lens, np.int32)).to(DEV)
    for pt in (0, 64):
        kp = torch.full((num_pages, hkv, 2048), fill, dtype=dt, device=DEV)
        vp = torch.full((num_pages, hkv, 2048), fill, dtype=dt, device=DEV)
        ks = torch.ones(hkv, dtype=torch.float32, device=DEV)
        vs = torch.ones(hkv, dtype=torch.float32, device=DEV)
        kv.ingest_layer(torch.from_numpy(rows_k.view(np.int16)).to(DEV),
                        torch.from_numpy(rows_v.view(np.int16)).to(DEV),
                        torch.from_numpy(start).to(DEV),
                        torch.from_numpy(np.array(prompt, np.int32)).to(DEV), btt, kp, vp,
                        max(lens), ks if fp8 else None, vs if fp8 else None, cache_dtype=cd)
        ab = torch.full((batch,), 0xA5, dtype=torch.uint8, device=DEV)
        kv.kv_verify_tags(d_tags, btt, d_exp, d_lens, ab)
        out = torch.full((batch, hq, 128), float("nan"), device=DEV)
        n = kv.paged_decode_attn_workspace_bytes(batch, hq, hkv, max(lens), pt, cache_dtype=cd)
        ws = torch.zeros(max(n, 256), dtype=torch.uint8, device=DEV)
        kv.paged_decode_attn_append(torch.from_numpy(q.view(np.int16)).to(DEV),
                                    torch.from_numpy(new_k.view(np.int16)).to(DEV),
                                    torch.from_numpy(new_v.view(np.int16)).to(DEV), kp, vp,
                                    ks if fp8 else None, vs if fp8 else None, btt, d_lens,
                                    max(lens), out, 0.0883883, workspace=ws, abort=ab,
                                    partition_tokens=pt, cache_dtype=cd)
        torch.cuda.synchronize()
        assert not ab.any().item()
        used = np.concatenate(ids)
        sel = torch.from_numpy(used.astype(np.int64)).to(DEV)
        kt, vt = kp[sel].cpu().numpy(), vp[sel].cpu().numpy()
        del kp, vp
        torch.cuda.empty_cache()
        if not fp8:
            kt, vt = kt.view(np.uint16), vt.view(np.uint16)
        kl, vl = helpers.tiles_to_logical(kt, "k", cache), helpers.tiles_to_logical(vt, "v", cache)
        if fp8:
            ks_o = ingest.scales_from_amax(ingest.amax_finite(rows_k))
            vs_o = ingest.scales_from_amax(ingest.amax_finite(rows_v))
            assert np.array_equal(ks.cpu().numpy().view(np.uint32), ks_o.view(np.uint32))
            assert np.array_equal(vs.cpu().numpy().view(np.uint32), vs_o.view(np.uint32))
        else:
            ks_o = vs_o = np.ones(hkv, np.float32)
        # the compact pool: request b's pages in order, its table remapped
        bt_c = np.full_like(bt, -1)
        pos = 0
        for b in range(batch):
            bt_c[b, :need[b]] = np.arange(pos, pos + need[b])
            pos += need[b]
            for pool, rows, new, sc in ((kl, rows_k, new_k, ks_o), (vl, rows_v, new_v, vs_o)):
                toks = np.concatenate([rows[start[b]:start[b] + prompt[b]], new[b][None]])
                want = e4m3.quantize(toks, sc[None, :, None]) if fp8 else toks
                got = pool[bt_c[b, :need[b]]].transpose(0, 2, 1, 3).reshape(-1, hkv, 128)
                assert np.array_equal(got[:lens[b]], want), f"{cache} p{pt}: codes of request {b}"
                # past the end: the ingest's zeros where it wrote the last page; the
                # fill where only the appended token reached it
                tail = 0 if -(-prompt[b] // 16) == need[b] else fill
                assert np.all(got[lens[b]:] == tail), \
                    f"{cache} p{pt}: tail of request {b}"
        want = paged.decode_attn(q, kl, vl, ks_o, vs_o, bt_c, np.array(lens, np.int32),
                                 0.0883883, cache)
        rel, mx = helpers.check_attention(out.cpu().numpy(), want,
                                          label=f"pool beyond 4 GiB {cache} p{pt}")
        say(f"pool of {num_pages} pages ({cache}, partitions {pt or 'auto'}): codes exact, "
            f"worst row rel_l2={rel:.2e}")


def test_one_million_token_request(kv):
    """One request of 1,000,000 tokens (62,500 pages per KV head, 1 GB per
    FP8 array), filled through the bulk append: the tag check splits its row
    over 31 workgroups (all matching -> 0; its last page's expected tag wrong
    -> 1 and an all-zero output), then one fused append + attention step in
    the shared kernel (62 automatic partitions of 16,384 tokens) and in the
    persistent kernel (1,954 partitions of 512). Each KV head's 8 query
    heads against the oracle over that head's codes as the launch left them;
    the appended token's codes are the oracle's."""
    hq, hkv, L = 64, 8, 1_000_000
    npg = -(-L // 16)
    num_pages = npg + 100
    rng = np.random.default_rng(1_000_000)
    bt = rng.permutation(num_pages)[:npg].astype(np.int32)[None]
    btt = torch.from_numpy(bt).to(DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    kp = torch.zeros((num_pages, hkv, 2048), dtype=torch.uint8, device=DEV)
    vp = torch.zeros_like(kp)
    k_rows = (torch.randn((L - 1, hkv, 128), generator=gen, device=DEV)).to(torch.bfloat16)
    v_rows = (torch.randn((L - 1, hkv, 128), generator=gen, device=DEV) * 0.5).to(torch.bfloat16)
    ks = (k_rows.abs().amax(dim=(0, 2)).float() / 448.0).contiguous()
    vs = (v_rows.abs().amax(dim=(0, 2)).float() / 448.0).contiguous()
    chunk = 1 << 16
    for t0 in range(0, L - 1, chunk):
        t1 = min(L - 1, t0 + chunk)
        pos = torch.arange(t0, t1, dtype=torch.int32, device=DEV)
        kv.kv_append_quant(k_rows[t0:t1].view(torch.int16), v_rows[t0:t1].view(torch.int16),
                           torch.zeros_like(pos), pos, btt, ks, vs, kp, vp)
    del k_rows, v_rows
    new_k = synth._f32_to_bf16_bits(rng.normal(0, 1, (1, hkv, 128)).astype(np.float32))
    new_v = synth._f32_to_bf16_bits(rng.normal(0, 0.5, (1, hkv, 128)).astype(np.float32))
    q = synth._f32_to_bf16_bits(rng.normal(0, 1, (1, hq, 128)).astype(np.float32))
    tags = rng.integers(0, 2 ** 32, num_pages, dtype=np.uint64).astype(np.uint32)
    exp = tags[bt].copy()
    d_tags = torch.from_numpy(tags.view(np.int32)).to(DEV)
    d_lens = torch.tensor([L], dtype=torch.int32, device=DEV)
    ws_v = torch.zeros(kv.kv_verify_tags_workspace_bytes(1, npg), dtype=torch.uint8, device=DEV)
    bad = exp.copy()
    bad[0, npg - 1] ^= 1
    ab = torch.full((1,), 0xA5, dtype=torch.uint8, device=DEV)
    kv.kv_verify_tags(d_tags, btt, torch.from_numpy(bad.view(np.int32)).to(DEV), d_lens, ab,
                      workspace=ws_v)
    torch.cuda.synchronize()
    assert ab.item() == 1 and int(ws_v.count_nonzero()) == 0
    ks_h, vs_h = ks.cpu().numpy(), vs.cpu().numpy()
    qt = torch.from_numpy(q.view(np.int16)).to(DEV)
    knt = torch.from_numpy(new_k.view(np.int16)).to(DEV)
    vnt = torch.from_numpy(new_v.view(np.int16)).to(DEV)
    out = torch.full((1, hq, 128), float("nan"), device=DEV)
    kp0, vp0 = kp.clone(), vp.clone()          # the aborted step must leave the pools as they are
    ws = torch.zeros(kv.paged_decode_attn_workspace_bytes(1, hq, hkv, L, 512), dtype=torch.uint8,
                     device=DEV)
    kv.paged_decode_attn_append(qt, knt, vnt, kp, vp, ks, vs, btt, d_lens, L, out, 0.0883883,
                                workspace=ws, abort=ab, partition_tokens=512)
    torch.cuda.synchronize()
    assert torch.all(out == 0).item() and torch.equal(kp, kp0) and torch.equal(vp, vp0)
    del kp0, vp0
    kv.kv_verify_tags(d_tags, btt, torch.from_numpy(exp.view(np.int32)).to(DEV), d_lens, ab,
                      workspace=ws_v)
    torch.cuda.synchronize()
    assert ab.item() == 0
    sel = torch.from_numpy(bt[0].astype(np.int64)).to(DEV)
    for pt in (0, 512):
        assert kv.paged_decode_attn_partition_tokens(1, hkv, L, pt) == (16384 if pt == 0 else 512)
        assert _uses_persistent_kernel(1, hkv, L, 16384 if pt == 0 else 512) == (pt == 512)
        out = torch.full((1, hq, 128), float("nan"), device=DEV)
        kv.paged_decode_attn_append(qt, knt, vnt, kp, vp, ks, vs, btt, d_lens, L, out, 0.0883883,
                                    workspace=ws, abort=ab, partition_tokens=pt)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        worst = 0.0
        for g in range(hkv):
            kc = helpers.tiles_to_logical(kp[sel, g].cpu().numpy(), "k", "fp8").reshape(-1, 128)[:L]
            vc = helpers.tiles_to_logical(vp[sel, g].cpu().numpy(), "v", "fp8").reshape(-1, 128)[:L]
            assert np.array_equal(kc[L - 1], e4m3.quantize(new_k[0, g], ks_h[g]))
            assert np.array_equal(vc[L - 1], e4m3.quantize(new_v[0, g], vs_h[g]))
            want = paged.attend_request(q[0, g * 8:(g + 1) * 8],
                                        e4m3.dequantize(kc, ks_h[g])[None],
                                        e4m3.dequantize(vc, vs_h[g])[None], 0.0883883)
            rel, _ = helpers.check_attention(got[:, g * 8:(g + 1) * 8], want[None],
                                             label=f"1M tokens p{pt} head {g}")
            worst = max(worst, rel)
        say(f"1,000,000-token request, partitions {pt or 'auto'}: worst row rel_l2={worst:.2e}")


def test_two_streams_at_once_equal_each_alone(kv):
    """The library keeps no state between calls beyond the caller's buffers:
    two batches decoded at the same time on two side streams (default
    priority), each with its own tag-check counters and split-K workspace,
    one through the persistent kernel and one through the shared kernel,
    give bit for bit what each gives alone on the default stream; three
    rounds, so the counters come back to zero in between."""
    rng = np.random.default_rng(31)
    jobs = []
    for lens, hq, pt in (((rng.integers(1, 3000, 40)).tolist(), 64, 64),
                         ((rng.integers(1, 9000, 6)).tolist(), 32, 0)):
        hkv = 8
        need = sum(max(1, -(-L // 16)) for L in lens)
        e = _edge_state(kv, "fp8", hq, hkv, lens, pool_pages=need + 8)
        batch = len(lens)
        width = max(3000, e["bt"].shape[1])              # rows wider than one check chunk
        bt = np.full((batch, width), -1, np.int32)
        bt[:, :e["bt"].shape[1]] = e["bt"]
        tags = rng.integers(0, 2 ** 32, need + 8, dtype=np.uint64).astype(np.uint32)
        exp = tags[np.clip(bt, 0, None)]
        msl = max(lens)
        n = kv.paged_decode_attn_workspace_bytes(batch, hq, hkv, msl, pt)
        jobs.append(dict(
            e=e, hq=hq, pt=pt, msl=msl, batch=batch,
            btt=torch.from_numpy(bt).to(DEV), tags=torch.from_numpy(tags.view(np.int32)).to(DEV),
            exp=torch.from_numpy(exp.view(np.int32)).to(DEV),
            lens=torch.from_numpy(np.array(lens, np.int32)).to(DEV),
            q=torch.from_numpy(e["q"].view(np.int16)).to(DEV),
            ws=torch.zeros(max(n, 256), dtype=torch.uint8, device=DEV),
            vws=torch.zeros(kv.kv_verify_tags_workspace_bytes(batch, width), dtype=torch.uint8,
                            device=DEV),
            ab=torch.zeros(batch, dtype=torch.uint8, device=DEV),
            out=torch.zeros((batch, hq, 128), dtype=torch.float32, device=DEV)))
    assert _uses_persistent_kernel(jobs[0]["batch"], 8, jobs[0]["msl"], 64)
    assert not _uses_persistent_kernel(jobs[1]["batch"], 8, jobs[1]["msl"],
                                       kv.paged_decode_attn_partition_tokens(
                                           jobs[1]["batch"], 8, jobs[1]["msl"], 0))

    def run(j, stream=None):
        kv.kv_verify_tags(j["tags"], j["btt"], j["exp"], j["lens"], j["ab"], workspace=j["vws"],
                          stream=stream)
        kv.paged_decode_attn(j["q"], j["e"]["kp"], j["e"]["vp"], j["e"]["kst"], j["e"]["vst"],
                             j["btt"], j["lens"], j["msl"], j["out"], 0.0883883,
                             workspace=j["ws"], abort=j["ab"], partition_tokens=j["pt"],
                             stream=stream)

    alone = []
    for j in jobs:
        run(j)
        torch.cuda.synchronize()
        assert not j["ab"].any().item()
        alone.append(j["out"].clone())
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rnd in range(3):
        for j in jobs:
            j["out"].fill_(float("nan"))
            j["ab"].fill_(0xA5)
        torch.cuda.synchronize()
        for _ in range(4):                   # the two streams' launches interleave
            for j, s in zip(jobs, streams):
                run(j, stream=s)
        torch.cuda.synchronize()
        for j, ref in zip(jobs, alone):
            assert not j["ab"].any().item()
            assert torch.equal(j["out"], ref), f"round {rnd}: hq {j['hq']}"
            assert int(j["vws"].count_nonzero()) == 0
    want = _edge_oracle(jobs[0]["e"], "fp8", jobs[0]["e"]["lens"])
    helpers.check_attention(alone[0].cpu().numpy(), want, label="two streams, job 0")
