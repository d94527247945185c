"""Full-size "needle" tests: one dominant token per (request, KV head) group.

At the headline and skewed workloads' full sizes, in the launch
configuration the benchmark times, every group gets one token whose key
points along that group's queries so strongly that the softmax puts all its
weight there: the group's output must then be that token's value. The needle
sits at the places where a misaddressed token would go unseen: the first and
last token of a page, of a page pair (the unit a wavefront streams), of a
partition and of a persistent-kernel piece, and the token the launch appends
itself. A dropped or misplaced needle gives the mean of thousands of values
instead, orders of magnitude outside the tolerance.

Also: the oracle output of one KV-head group of every request of the headline
batch's layer 0, regenerated request by request.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import e4m3, paged
from synth.device import DeviceState
from tests import helpers
from tests import wave_split_model as ws
from tests.gpu_harness import DEV, say, sm_scale_for, workspace

pytestmark = pytest.mark.gpu
P = 16


@pytest.fixture(scope="module")
def kv():
    import fp8_e4m3_paged_amd as k
    k.load()
    return k


def _needle_round(kv, st, q, kn, vn, needles, partition_tokens, rng, label):
    """Plant needles {(b, g): t}, run the fused step of layer 0, check every
    group, restore the pool. A needle at t = L - 1 arrives through the new
    token (the launch writes it); any other through the pool."""
    wl = st.wl
    G = wl.num_q_heads // wl.num_kv_heads
    L = wl.seq_lens_at(0)
    koff = torch.from_numpy(helpers.OFFSETS[("k", "fp8")].astype(np.int64)).to(DEV)
    voff = torch.from_numpy(helpers.OFFSETS[("v", "fp8")].astype(np.int64)).to(DEV)
    qh = q.view(torch.int16).cpu().numpy().view(np.uint16)
    kn_r = kn.clone()
    vn_r = vn.clone()
    expect = {}
    saved = []
    for (b, g), t in needles.items():
        sign = (qh[b, g * G] & 0x8000) != 0                       # the group's q direction
        v_codes = rng.integers(0, 0x7E, 128).astype(np.uint8) | (rng.integers(0, 2, 128) << 7).astype(np.uint8)
        vs = np.float32(st.v_scale_host[0][g])
        if t == L[b] - 1:
            kbits = np.where(sign, 0xC61C, 0x461C).astype(np.uint16)     # -+10000 in bf16
            vval = e4m3.dequantize(v_codes, vs).astype(np.float32)        # exact in fp32
            vbits = synth._f32_to_bf16_bits(vval)                          # nearest bf16
            kn_r[b, g] = torch.from_numpy(kbits.view(np.int16)).to(DEV)
            vn_r[b, g] = torch.from_numpy(vbits.view(np.int16)).to(DEV)
            expect[(b, g)] = e4m3.dequantize(e4m3.quantize(vbits, vs), vs)
            continue
        page = int(wl.block_table[b, t // P])
        slot = t % P
        kc = torch.from_numpy(np.where(sign, 0xFE, 0x7E).astype(np.uint8)).to(DEV)    # -+448
        ki = koff[slot]
        vi = voff[slot]
        saved.append((page, g, ki, vi, st.k_pool[0][page, g, ki].clone(),
                      st.v_pool[0][page, g, vi].clone()))
        st.k_pool[0][page, g, ki] = kc
        st.v_pool[0][page, g, vi] = torch.from_numpy(v_codes).to(DEV)
        expect[(b, g)] = e4m3.dequantize(v_codes, vs)
    out = torch.full((wl.batch, wl.num_q_heads, wl.head_dim), float("nan"), device=DEV)
    seq = st.seq_lens(0)
    kv.kv_verify_tags(st.pool_tags, st.block_table, st.expected_tags, seq, st.abort)
    kv.paged_decode_attn_append(q, kn_r, vn_r, st.k_pool[0], st.v_pool[0], st.k_scale[0],
                                st.v_scale[0], st.block_table, seq, wl.max_seq_len, out,
                                sm_scale_for(wl), workspace=workspace(wl, partition_tokens),
                                abort=st.abort, partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    assert not st.abort.any().item()
    o = out.cpu().numpy()
    got = np.stack([o[b, g * G:(g + 1) * G] for (b, g) in needles])
    want = np.stack([np.repeat(expect[(b, g)][None], G, axis=0) for (b, g) in needles])
    rel, mx = helpers.check_attention(got, want, label=label)
    say(f"{label}: {len(needles)} needles, worst row rel_l2={rel:.2e} max_abs={mx:.2e}")
    for page, g, ki, vi, k0, v0 in saved:
        st.k_pool[0][page, g, ki] = k0
        st.v_pool[0][page, g, vi] = v0


def _aligned_queries(wl, q):
    """Every query head of a group gets the group's first head's vector with
    each element replaced by +-1 (its sign): score of a +-448 s_K needle =
    sm_scale * 128 * 448 s_K, far above any other token's."""
    G = wl.num_q_heads // wl.num_kv_heads
    qh = q.view(torch.int16).cpu().numpy().view(np.uint16).copy()
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            sign = qh[b, g * G] & 0x8000
            qh[b, g * G:(g + 1) * G] = (0x3F80 | sign)[None, :]
    return torch.from_numpy(qh.view(np.int16)).to(DEV).view(torch.bfloat16)


def test_needles_batch64_shared_kernel(kv):
    """The headline batch (one partition per group, four wavefronts taking
    page pairs round-robin), layer 0, fused append + attention."""
    wl = synth.batch64_ctx8k(max_steps=1)
    say("needles batch64: building layer 0 (batch 64, ctx 8192+U[0,1000])")
    st = DeviceState(wl, kv, cache="fp8", device=DEV, layers=[0])
    q, kn, vn = st.step_layer_inputs(0, 0)
    q = _aligned_queries(wl, q)
    L = wl.seq_lens_at(0)
    rng = np.random.default_rng(64)

    def classes(b):
        n = -(-int(L[b]) // P)
        last_pair = 2 * ((n - 1) // 2)
        return [0, 15, 16, 31, 32, 63, 64, 127, 128, 16 * last_pair, 16 * (n - 1),
                int(L[b]) - 2, int(L[b]) - 1, int(rng.integers(0, int(L[b])))]

    groups = [(b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)]
    n_cls = len(classes(0))
    for rnd in range(2):
        needles = {(b, g): classes(b)[(b * 8 + g + rnd * 7) % n_cls] for (b, g) in groups}
        _needle_round(kv, st, q, kn, vn, needles, 0, rng, f"needles batch64 round {rnd}")


def test_needles_skewed16_persistent_kernel(kv):
    """The skewed workload (lengths to 131,072) in 512-token partitions: the
    persistent kernel with its even split; needles at piece and partition
    boundaries, placed with the host model of the split."""
    wl = synth.skewed_16req(max_steps=1)
    say("needles skewed16: building (batch 16, lengths to 131072)")
    st = DeviceState(wl, kv, cache="fp8", device=DEV)
    q, kn, vn = st.step_layer_inputs(0, 0)
    q = _aligned_queries(wl, q)
    L = wl.seq_lens_at(0)
    assert ws.uses_wave_kernel(wl.batch, wl.num_kv_heads, wl.max_seq_len, 512)
    pieces = ws.split(L.tolist(), wl.num_kv_heads, 512, wl.max_seq_len,
                      wl.block_table.shape[1])
    starts, ends = {}, {}
    for pc in pieces:
        starts.setdefault((pc.b, pc.g), []).append(16 * pc.k0)
        ends.setdefault((pc.b, pc.g), []).append(min(16 * pc.k_end, int(L[pc.b])) - 1)
    rng = np.random.default_rng(16)

    def classes(b, g):
        n_tok = int(L[b])
        parts = [t for t in range(512, n_tok, 512)]
        cand = [
            rng.choice(starts[(b, g)]), rng.choice(ends[(b, g)]),
            rng.choice(parts) if parts else 0, (rng.choice(parts) - 1) if parts else 15,
            0, n_tok - 1, n_tok - 2, 16 * int(rng.integers(0, -(-n_tok // P))),
        ]
        return [int(min(max(c, 0), n_tok - 1)) for c in cand]

    groups = [(b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)]
    for rnd in range(4):
        needles = {}
        for (b, g) in groups:
            cls = classes(b, g)
            needles[(b, g)] = cls[(b * 8 + g + rnd * 3) % len(cls)]
        _needle_round(kv, st, q, kn, vn, needles, 512, rng, f"needles skewed16 round {rnd}")


def test_batch64_every_request_one_group_against_oracle(kv):
    """Layer 0 of the headline batch, fused step as benchmarked: for every
    request, KV head b % 8 regenerated on the host, its codes bit for bit and
    its 8 query heads within the tolerance."""
    wl = synth.batch64_ctx8k(max_steps=1)
    st = DeviceState(wl, kv, cache="fp8", device=DEV, layers=[0])
    q, kn, vn = st.step_layer_inputs(0, 0)
    out = torch.full((wl.batch, wl.num_q_heads, wl.head_dim), float("nan"), device=DEV)
    seq = st.seq_lens(0)
    kv.kv_verify_tags(st.pool_tags, st.block_table, st.expected_tags, seq, st.abort)
    kv.paged_decode_attn_append(q, kn, vn, st.k_pool[0], st.v_pool[0], st.k_scale[0],
                                st.v_scale[0], st.block_table, seq, wl.max_seq_len, out,
                                sm_scale_for(wl), workspace=workspace(wl, 0), abort=st.abort)
    torch.cuda.synchronize()
    assert not st.abort.any().item()
    o = out.cpu().numpy()
    qb = q.view(torch.int16).cpu().numpy().view(np.uint16)
    G = wl.num_q_heads // wl.num_kv_heads
    L = wl.seq_lens_at(0)
    worst = 0.0
    for b in range(wl.batch):
        g = b % wl.num_kv_heads
        n = -(-int(L[b]) // P)
        ids = torch.from_numpy(wl.block_table[b, :n].astype(np.int64)).to(DEV)
        kt = st.k_pool[0][ids, g].cpu().numpy()
        vt = st.v_pool[0][ids, g].cpu().numpy()
        kd = helpers.tiles_to_logical(kt, "k", "fp8").reshape(-1, 128)[:L[b]]
        vd = helpers.tiles_to_logical(vt, "v", "fp8").reshape(-1, 128)[:L[b]]
        kc = e4m3.quantize(wl.kv_bits_head(0, "k", b, g, 0, int(L[b])), st.k_scale_host[0][g])
        vc = e4m3.quantize(wl.kv_bits_head(0, "v", b, g, 0, int(L[b])), st.v_scale_host[0][g])
        assert np.array_equal(kd, kc), f"K codes of request {b} head {g}"
        assert np.array_equal(vd, vc), f"V codes of request {b} head {g}"
        Kd = e4m3.dequantize(kc, st.k_scale_host[0][g])[None]
        Vd = e4m3.dequantize(vc, st.v_scale_host[0][g])[None]
        want = paged.attend_request(qb[b, g * G:(g + 1) * G], Kd, Vd, sm_scale_for(wl))
        rel, _ = helpers.check_attention(o[b:b + 1, g * G:(g + 1) * G], want[None],
                                         label=f"batch64 request {b} group {g}")
        worst = max(worst, rel)
    say(f"batch64 layer 0: one group of each of 64 requests, worst row rel_l2={worst:.2e}")
