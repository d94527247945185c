"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses, on sampled outputs the oracle recomputes one request (or one
KV-head group) at a time from the seeded generator.

For each sample: the request's pool codes (its pages, read back from the GPU
and mapped through the documented tile layout) are compared bit-exactly with
the oracle's codes, then the attention output of that request is compared
within the tolerance. Abort masks are compared whole. One layer of the
headline, skewed and 32-request batches (both caches) are also checked
whole: every code of the pools the launch left, and every output against the
oracle over those pools.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import synth
from oracle import e4m3, paged
from synth.device import DeviceState
from tests import helpers
from tests.gpu_harness import DEV, gpu_step, say, sm_scale_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kv():
    import fp8_e4m3_paged_amd as k
    k.load()
    return k


def _device_request_pages(st, layer, b, L):
    """Device tiles of request b's first ceil(L/16) pages -> host arrays."""
    n = -(-L // 16)
    ids = torch.from_numpy(st.wl.block_table[b, :n].astype(np.int64)).to(DEV)
    kt = st.k_pool[layer][ids].cpu().numpy()
    vt = st.v_pool[layer][ids].cpu().numpy()
    if st.cache == "bf16":
        kt, vt = kt.view(np.uint16), vt.view(np.uint16)
    return kt, vt


def _check_group(st, layer, b, g, step, q_bits, out, label):
    """Oracle for KV-head group g of request b, regenerated alone; codes of
    that head compared bit-exactly, then the group's G query heads."""
    wl = st.wl
    L = int(wl.seq_lens_at(step)[b])
    G = wl.num_q_heads // wl.num_kv_heads
    kb = wl.kv_bits_head(layer, "k", b, g, 0, L)
    vb = wl.kv_bits_head(layer, "v", b, g, 0, L)
    kt, vt = _device_request_pages(st, layer, b, L)
    kd = helpers.tiles_to_logical(kt[:, g], "k", st.cache).reshape(-1, 128)[:L]
    vd = helpers.tiles_to_logical(vt[:, g], "v", st.cache).reshape(-1, 128)[:L]
    if st.cache == "fp8":
        kc = e4m3.quantize(kb, st.k_scale_host[layer][g])
        vc = e4m3.quantize(vb, st.v_scale_host[layer][g])
        assert np.array_equal(kd, kc), f"{label}: K codes of request {b} head {g}"
        assert np.array_equal(vd, vc), f"{label}: V codes of request {b} head {g}"
        Kd = e4m3.decode(kc)[None] * np.float64(st.k_scale_host[layer][g])
        Vd = e4m3.decode(vc)[None] * np.float64(st.v_scale_host[layer][g])
    else:
        assert np.array_equal(kd, kb) and np.array_equal(vd, vb), f"{label}: bf16 pages"
        Kd = e4m3.bf16_bits_to_f64(kb)[None]
        Vd = e4m3.bf16_bits_to_f64(vb)[None]
    want = paged.attend_request(q_bits[b, g * G:(g + 1) * G], Kd, Vd, sm_scale_for(wl))
    rel, mx = helpers.check_attention(out[b:b + 1, g * G:(g + 1) * G], want[None],
                                      label=f"{label} b={b} g={g} L={L}")
    say(f"{label}: layer {layer} request {b} (L={L}) group {g}: rel_l2={rel:.2e} max_abs={mx:.2e}")


def test_batch64_ctx8k_full_size(kv):
    wl = synth.batch64_ctx8k(max_steps=2)
    say("batch64: building 8-layer FP8 pools (batch 64, ctx 8192+U[0,1000])")
    st = DeviceState(wl, kv, cache="fp8", device=DEV)
    # verify on, automatic partition, fused append + attention: as benchmarked
    ab, outs, inputs = gpu_step(st, 0, fused=True)
    assert not ab.any()
    L = wl.seq_lens_at(0)
    samples = [(int(np.argmax(L)), 7, 5), (int(np.argmin(L)), 0, 0), (17, 3, 2), (40, 5, 7)]
    for b, layer, g in samples:
        _check_group(st, layer, b, g, 0, inputs[layer][0], outs[layer], "batch64")
    for layer in st.layers:
        assert np.all(np.isfinite(outs[layer]))


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_uniform_32req_full_size(kv, cache):
    wl = synth.uniform_32req(max_steps=1)
    say(f"uniform32/{cache}: building 8-layer pools (batch 32, ctx 8192)")
    st = DeviceState(wl, kv, cache=cache, device=DEV)
    ab, outs, inputs = gpu_step(st, 0)
    assert not ab.any()
    for b, layer, g in [(0, 0, 0), (31, 7, 7), (13, 4, 3)]:
        _check_group(st, layer, b, g, 0, inputs[layer][0], outs[layer], f"uniform32/{cache}")


def test_uniform_32req_fp8_equals_quantized_bf16(kv):
    """Same seeded values in both caches: the FP8 output approximates the BF16
    one within the error FP8 storage itself introduces (loose), while each
    matches its own oracle tightly (above)."""
    wl = synth.uniform_32req(max_steps=1)
    st8 = DeviceState(wl, kv, cache="fp8", device=DEV, layers=[0])
    _, o8, _ = gpu_step(st8, 0)
    del st8
    torch.cuda.empty_cache()
    st16 = DeviceState(wl, kv, cache="bf16", device=DEV, layers=[0])
    _, o16, _ = gpu_step(st16, 0)
    err = np.linalg.norm(o8[0] - o16[0]) / np.linalg.norm(o16[0])
    say(f"uniform32: FP8 vs BF16 cache output rel_l2 = {err:.3e}")
    assert 1e-4 < err < 0.2


def test_skewed_16req_split_k_and_churn(kv):
    wl = synth.skewed_16req(max_steps=2)
    stale = wl.notes["churn_stale"]
    say(f"skewed16: lengths {sorted(wl.seq_lens_at(0).tolist())}, stale after churn {stale}")
    st = DeviceState(wl, kv, cache="fp8", device=DEV)
    pt = wl.partition_tokens
    ab0, outs0, inputs0 = gpu_step(st, 0, partition_tokens=pt)
    assert not ab0.any()
    L0 = wl.seq_lens_at(0)
    longest = int(np.argmax(L0))
    shortest = int(np.argmin(L0))
    for b, g in [(longest, 1), (shortest, 6), (5, 3)]:
        _check_group(st, 0, b, g, 0, inputs0[0][0], outs0[0], "skewed16 step 0")
    # between steps: 10% of the pages are freed and reallocated with a tag
    # bump; the two stale requests keep their old expectations
    wl.notes["churn_step"] = 1
    wl.apply_churn(np.random.default_rng(wl.notes["churn_rng_seed"]), 0.10, stale)
    st.upload_tags()
    ab1, outs1, inputs1 = gpu_step(st, 1, partition_tokens=pt, fused=True)
    want = paged.verify_tags(wl.pool_tags, wl.block_table, wl.expected_tags, wl.seq_lens_at(1), 16)
    assert np.array_equal(ab1, want)
    assert sorted(np.flatnonzero(ab1).tolist()) == sorted(stale)
    for b in stale:
        assert np.all(outs1[0][b] == 0.0)
    ok = [b for b in range(wl.batch) if b not in stale]
    for b, g in [(ok[0], 0), (ok[-1], 4)]:
        _check_group(st, 0, b, g, 1, inputs1[0][0], outs1[0], "skewed16 step 1")


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _logical_threaded(tiles, kind, cache):
    """tiles_to_logical over a whole layer's pool, in page chunks on threads."""
    out = np.empty(tiles.shape[:-1] + (16, 128), tiles.dtype)
    bounds = np.linspace(0, tiles.shape[0], 65).astype(np.int64)

    def conv(i):
        a, b = bounds[i], bounds[i + 1]
        out[a:b] = helpers.tiles_to_logical(tiles[a:b], kind, cache)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(conv, range(64)))
    return out


@pytest.mark.parametrize("config,cache", [("batch64", "fp8"), ("batch64", "bf16"),
                                          ("skewed16", "fp8"), ("skewed16", "bf16"),
                                          ("uniform32", "fp8"), ("uniform32", "bf16")])
def test_every_output_of_a_full_size_layer(kv, config, cache):
    """Every output of one full-size layer, not a sample, with either cache:
    the headline batch (64 requests, one partition each in 4-wave
    workgroups, as benchmarked), the skewed batch (512-token partitions in
    the persistent kernel, then the reduce) and the 32-request batch (8-wave
    workgroups), each as one fused
    append + attention launch after the tag check. The whole layer's pools
    are read back after the launch, and the oracle attends every request over
    them (the same dequantized inputs, the token appended by the launch
    included; one request per thread, BLAS on one thread each); each
    (request, query head) row must meet the tolerance. Every code of every
    request's tokens, the initial fill and the appended token, is the oracle's
    encoding of its seeded bf16 row (BF16 cache: the row itself), so the pages
    the attention read are checked whole too."""
    make = {"batch64": synth.batch64_ctx8k, "skewed16": synth.skewed_16req,
            "uniform32": synth.uniform_32req}[config]
    wl = make(max_steps=1)
    st = DeviceState(wl, kv, cache=cache, device=DEV, layers=[0])
    pt = wl.partition_tokens if config == "skewed16" else 0
    ab, outs, inputs = gpu_step(st, 0, partition_tokens=pt, fused=True)
    assert not ab.any()
    q_bits, kn, vn = inputs[0]
    kt, vt = st.k_pool[0].cpu().numpy(), st.v_pool[0].cpu().numpy()
    if cache == "bf16":
        kt, vt = kt.view(np.uint16), vt.view(np.uint16)
    kl, vl = _logical_threaded(kt, "k", cache), _logical_threaded(vt, "v", cache)
    L = wl.seq_lens_at(0).astype(np.int32)
    ks, vs = st.k_scale_host[0], st.v_scale_host[0]
    # the token each request appended this step (position L - 1)
    for b in range(wl.batch):
        t = int(L[b]) - 1
        page = int(wl.block_table[b, t // 16])
        want_k = e4m3.quantize(kn[b], ks[:, None]) if cache == "fp8" else kn[b]
        want_v = e4m3.quantize(vn[b], vs[:, None]) if cache == "fp8" else vn[b]
        assert np.array_equal(kl[page, :, t % 16], want_k), f"K row {b}"
        assert np.array_equal(vl[page, :, t % 16], want_v), f"V row {b}"

    # every code of every request's tokens (the initial fill and the appended
    # token) against the oracle's encoding of the seeded bf16 rows
    def codes_ok(bg):
        b, g = bg
        n = int(L[b])
        ids = wl.block_table[b, :-(-n // 16)]
        for kind, pool, sc in (("k", kl, ks), ("v", vl, vs)):
            bits = wl.kv_bits_head(0, kind, b, g, 0, n)
            want_c = e4m3.quantize(bits, sc[g]) if cache == "fp8" else bits
            if not np.array_equal(pool[ids, g].reshape(-1, 128)[:n], want_c):
                return (b, g, kind)
        return None

    groups = [(b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)]
    with threadpool_limits(1), ThreadPoolExecutor(_threads()) as ex:
        bad = [r for r in ex.map(codes_ok, groups) if r is not None]
    assert not bad, f"{config} {cache}: codes differ for (request, head, K|V) {bad[:8]}"
    sm = sm_scale_for(wl)
    with threadpool_limits(1), ThreadPoolExecutor(_threads()) as ex:
        want = np.stack(list(ex.map(
            lambda b: paged.decode_attn_request(b, q_bits, kl, vl, ks, vs, wl.block_table, L,
                                                sm, cache), range(wl.batch))))
    rel, mx = helpers.check_attention(outs[0], want, label=f"{config} {cache} every output")
    say(f"{config} {cache}: all {wl.batch} x {wl.num_q_heads} rows of layer 0, worst rel_l2={rel:.2e} "
        f"max_abs={mx:.2e}")


def test_every_output_after_churn(kv):
    """The skewed batch's second step after the churn (10% of pages freed
    and reallocated with tag bumps; two requests keep stale mappings), as one
    fused launch after the tag check: the mask is exactly the two stale
    requests, their rows are zero and their append slots untouched, every
    other request's appended codes are the oracle's, and every output of the
    others is within the tolerance of the oracle over the pools the launch
    left."""
    wl = synth.skewed_16req(max_steps=2)
    stale = wl.notes["churn_stale"]
    st = DeviceState(wl, kv, cache="fp8", device=DEV, layers=[0])
    pt = wl.partition_tokens
    ab0, _, _ = gpu_step(st, 0, partition_tokens=pt, fused=True)
    assert not ab0.any()
    wl.notes["churn_step"] = 1
    wl.apply_churn(np.random.default_rng(wl.notes["churn_rng_seed"]), 0.10, stale)
    st.upload_tags()
    L = wl.seq_lens_at(1).astype(np.int32)
    # the stale requests' target slots before the step
    before = {}
    for b in stale:
        t = int(L[b]) - 1
        page = int(wl.block_table[b, t // 16])
        before[b] = (page, st.k_pool[0][page].cpu().numpy().copy(),
                     st.v_pool[0][page].cpu().numpy().copy())
    ab, outs, inputs = gpu_step(st, 1, partition_tokens=pt, fused=True)
    assert sorted(np.flatnonzero(ab).tolist()) == sorted(stale)
    for b in stale:
        page, k0, v0 = before[b]
        assert np.array_equal(st.k_pool[0][page].cpu().numpy(), k0), f"stale {b} wrote K"
        assert np.array_equal(st.v_pool[0][page].cpu().numpy(), v0), f"stale {b} wrote V"
    q_bits, kn, vn = inputs[0]
    kl = _logical_threaded(st.k_pool[0].cpu().numpy(), "k", "fp8")
    vl = _logical_threaded(st.v_pool[0].cpu().numpy(), "v", "fp8")
    ks, vs = st.k_scale_host[0], st.v_scale_host[0]
    for b in range(wl.batch):
        if b in stale:
            continue
        t = int(L[b]) - 1
        page = int(wl.block_table[b, t // 16])
        assert np.array_equal(kl[page, :, t % 16], e4m3.quantize(kn[b], ks[:, None])), f"K row {b}"
        assert np.array_equal(vl[page, :, t % 16], e4m3.quantize(vn[b], vs[:, None])), f"V row {b}"
    abort = np.zeros(wl.batch, np.uint8)
    abort[list(stale)] = 1
    sm = sm_scale_for(wl)
    with threadpool_limits(1), ThreadPoolExecutor(_threads()) as ex:
        want = np.stack(list(ex.map(
            lambda b: paged.decode_attn_request(b, q_bits, kl, vl, ks, vs, wl.block_table, L,
                                                sm, "fp8", abort), range(wl.batch))))
    rel, mx = helpers.check_attention(outs[0], want, zero_rows=list(stale),
                                      label="skewed16 after churn, every output")
    say(f"skewed16 after churn: stale {sorted(stale)} zero and unwritten; the other "
        f"{wl.batch - len(stale)} x {wl.num_q_heads} rows worst rel_l2={rel:.2e} max_abs={mx:.2e}")
