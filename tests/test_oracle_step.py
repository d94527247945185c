"""Pins for the oracle's whole decode step and for dequantize-on-read (CPU only).

``oracle.paged.decode_step`` composes the tag check, the append and the
attention in the order the pages require: the check runs before any decode
read, and a mismatch aborts only that request (remio.ai/it "Il serving di
modelli più piccoli di Cloudflare riduce la memoria, ma la sicurezza diventa
la prova decisiva", section "Cosa ha cambiato Cloudflare per Kimi e GLM").
Here it is tied to things outside itself:

* a pure-Python step (scalar loops, the scalar brute-force encoder and the
  brute-force attention) on tiny states, several layers, FP8 and BF16;
* closed forms: a one-token request returns its own appended value; a new
  key that dominates every score makes the output its value, which is only
  possible if the append lands before the same step's read;
* the abort semantics: a stale request's bytes stay as they were in every
  layer, its output is zero, the other requests do not see it; with the
  no-op tracker nothing is aborted and the stale request is written and read.

``oracle.e4m3.dequantize`` is pinned by the OCP specification's stated values
times the scale and by the half-step bound of round-to-nearest.
"""

import math
import os

import numpy as np
import pytest

import synth
from oracle import e4m3, paged
from tests.test_oracle_paged import brute_force_attention

P = 16
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "ocp_e4m3_values.txt")


# ---------------------------------------------------------------------------
# dequantize
# ---------------------------------------------------------------------------
def _golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                code, val = line.split()
                rows.append((int(code, 16), float(val)))
    return rows


@pytest.mark.parametrize("scale", [1.0, 0.5, 3.0 / 448.0, 0.0123, 7.25])
def test_dequantize_reads_the_ocp_values_times_the_scale(scale):
    s = np.float32(scale)
    for code, val in _golden():
        got = e4m3.dequantize(np.array([code], np.uint8), s)[0]
        if math.isnan(val):
            assert math.isnan(got)
        else:
            assert got == val * float(s), (hex(code), got, val)
            assert math.copysign(1.0, got) == math.copysign(1.0, val)


def test_dequantize_of_quantize_is_within_half_a_step():
    """Round-to-nearest with 3 mantissa bits: a normal quotient comes back
    within 2^-4 of itself (relative), a subnormal one within 2^-10 absolute,
    and anything at or beyond 448 comes back as +-448 (saturation)."""
    rng = np.random.default_rng(31)
    x = synth._f32_to_bf16_bits(rng.standard_normal(200_000).astype(np.float32) *
                                np.float32(3.0))
    for s in np.float32([1.0, 0.01, 4.33 / 448.0, 1e-3, 0.5]):
        xv = e4m3.bf16_bits_to_f64(x)
        back = e4m3.dequantize(e4m3.quantize(x, s), s)
        y = xv / np.float64(s)
        normal = (np.abs(y) >= 2.0 ** -6) & (np.abs(y) < 448.0)
        sub = np.abs(y) < 2.0 ** -6
        sat = np.abs(y) >= 448.0
        assert normal.any() and sub.any()
        assert np.all(np.abs(back[normal] - xv[normal]) <= 2.0 ** -4 * np.abs(xv[normal]))
        assert np.all(np.abs(back[sub] - xv[sub]) <= 2.0 ** -10 * np.float64(s))
        assert np.all(back[sat] == np.sign(xv[sat]) * 448.0 * np.float64(s))


# ---------------------------------------------------------------------------
# whole steps
# ---------------------------------------------------------------------------
def step_state(rng, lens, hq=4, hkv=2, d=8, layers=2, cache="fp8", pool_pages=24):
    """A multi-layer paged state whose requests attend over ``lens`` tokens
    after this step's append (token L - 1 is the new one; its slot holds
    junk before the step)."""
    batch = len(lens)
    need = [max(1, -(-L // P)) for L in lens]
    perm = rng.permutation(pool_pages)
    bt = np.full((batch, max(need) + 1), -1, np.int32)
    off = 0
    for b in range(batch):
        bt[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    tags = rng.integers(0, 2 ** 32, pool_pages, dtype=np.uint64).astype(np.uint32)
    exp = np.zeros_like(bt, dtype=np.uint32)
    exp[bt >= 0] = tags[bt[bt >= 0]]
    st = dict(pool_tags=tags, block_table=bt, expected_tags=exp,
              seq_lens=np.array(lens, np.int32), page_size=P,
              k_pool=[], v_pool=[], k_scale=[], v_scale=[])
    q, kn, vn = [], [], []
    for _ in range(layers):
        if cache == "fp8":
            kp = rng.integers(0, 256, (pool_pages, hkv, P, d)).astype(np.uint8)
            vp = rng.integers(0, 256, (pool_pages, hkv, P, d)).astype(np.uint8)
            kp[(kp & 0x7F) == 0x7F] = 0x35          # no NaN codes in what is read
            vp[(vp & 0x7F) == 0x7F] = 0x35
        else:
            kp = synth._f32_to_bf16_bits(rng.normal(0, 1, (pool_pages, hkv, P, d))
                                         .astype(np.float32))
            vp = synth._f32_to_bf16_bits(rng.normal(0, 1, (pool_pages, hkv, P, d))
                                         .astype(np.float32))
        st["k_pool"].append(kp)
        st["v_pool"].append(vp)
        st["k_scale"].append(rng.uniform(0.002, 0.02, hkv).astype(np.float32))
        st["v_scale"].append(rng.uniform(0.002, 0.02, hkv).astype(np.float32))
        q.append(synth._f32_to_bf16_bits(rng.normal(0, 1, (batch, hq, d)).astype(np.float32)))
        kn.append(synth._f32_to_bf16_bits(rng.normal(0, 0.6, (batch, hkv, d)).astype(np.float32)))
        vn.append(synth._f32_to_bf16_bits(rng.normal(0, 0.6, (batch, hkv, d)).astype(np.float32)))
    return st, q, kn, vn


def copy_state(st):
    c = dict(st)
    for key in ("k_pool", "v_pool", "k_scale", "v_scale"):
        c[key] = [a.copy() for a in st[key]]
    for key in ("pool_tags", "block_table", "expected_tags", "seq_lens"):
        c[key] = st[key].copy()
    return c


def _bf(bits):
    return float(np.array([int(bits) << 16], np.uint32).view(np.float32)[0])


def brute_force_step(st, q, kn, vn, sm, cache, verify=True):
    """The step in scalar Python: the check as nested loops, the append
    through the scalar brute-force encoder, the attention through the
    pure-Python loops of the attention pin. Returns (abort, outs, pools)."""
    bt, lens = st["block_table"], st["seq_lens"]
    batch = len(lens)
    num_pages = st["k_pool"][0].shape[0]
    abort = [0] * batch
    if verify:
        for b in range(batch):
            L = int(lens[b])
            npg = (L + P - 1) // P
            if L < 0 or npg > bt.shape[1]:
                abort[b] = 1
                continue
            for j in range(npg):
                page = int(bt[b][j])
                if not (0 <= page < num_pages) or int(st["pool_tags"][page]) != int(
                        st["expected_tags"][b][j]):
                    abort[b] = 1
    pools, outs = [], []
    for layer in range(len(q)):
        kp = st["k_pool"][layer].copy()
        vp = st["v_pool"][layer].copy()
        hkv, d = kp.shape[1], kp.shape[3]
        for b in range(batch):
            L = int(lens[b])
            if abort[b] or L < 1:
                continue
            t = L - 1
            page, slot = int(bt[b][t // P]), t % P
            for g in range(hkv):
                for i in range(d):
                    if cache == "fp8":
                        ks = float(np.float32(st["k_scale"][layer][g]))
                        vs = float(np.float32(st["v_scale"][layer][g]))
                        kp[page][g][slot][i] = e4m3.encode_bruteforce(_bf(kn[layer][b][g][i]) / ks)
                        vp[page][g][slot][i] = e4m3.encode_bruteforce(_bf(vn[layer][b][g][i]) / vs)
                    else:
                        kp[page][g][slot][i] = kn[layer][b][g][i]
                        vp[page][g][slot][i] = vn[layer][b][g][i]
        att = dict(q=q[layer], kp=kp, vp=vp, bt=bt, lens=lens, ks=st["k_scale"][layer],
                   vs=st["v_scale"][layer])
        out = brute_force_attention(att, sm, cache)
        for b in range(batch):
            if abort[b]:
                out[b] = 0.0
        outs.append(out)
        pools.append((kp, vp))
    return np.array(abort, np.uint8), outs, pools


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_step_matches_pure_python_bruteforce(cache):
    rng = np.random.default_rng(41)
    st, q, kn, vn = step_state(rng, [37, 1, 16, 17, 33], cache=cache, layers=2)
    stale_b, stale_j = 3, 1
    st["expected_tags"][stale_b, stale_j] ^= np.uint32(1 << 9)   # request 3 is stale
    sm = 1 / math.sqrt(8)
    want_ab, want_out, want_pools = brute_force_step(st, q, kn, vn, sm, cache)
    assert want_ab.tolist() == [0, 0, 0, 1, 0]
    got_st = copy_state(st)
    ab, outs = paged.decode_step(got_st, q, kn, vn, sm, cache=cache)
    assert np.array_equal(ab, want_ab)
    for layer in range(2):
        assert np.array_equal(got_st["k_pool"][layer], want_pools[layer][0])
        assert np.array_equal(got_st["v_pool"][layer], want_pools[layer][1])
        assert np.max(np.abs(outs[layer] - want_out[layer])) <= 1e-12


def _align_group_with_new_key(q, kn, layer, b, g, group):
    """Give every query head of group g of request b the same vector u and
    make request b's new key +-big along sign(u) (it saturates to +-448 s)."""
    u = q[layer][b, g * group]
    for h in range(g * group, (g + 1) * group):
        q[layer][b, h] = u
    sign = np.where(u & 0x8000, -1.0, 1.0).astype(np.float32)
    kn[layer][b, g] = synth._f32_to_bf16_bits(sign * np.float32(1e4))


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_step_reads_the_token_it_appends(cache):
    """A new key far larger than every other along q: the softmax puts all
    its weight there, so the output equals that token's value (dequantized),
    which holds only if the append precedes the read within the step."""
    rng = np.random.default_rng(42)
    lens = [40, 19, 64]
    st, q, kn, vn = step_state(rng, lens, hq=4, hkv=2, d=32, layers=1, cache=cache,
                               pool_pages=16)
    group = 2
    for b in range(3):
        for g in range(2):
            _align_group_with_new_key(q, kn, 0, b, g, group)
    ab, outs = paged.decode_step(st, q, kn, vn, 0.5, cache=cache)
    assert not ab.any()
    for b in range(3):
        for g in range(2):
            if cache == "fp8":
                s = np.float32(st["v_scale"][0][g])
                v = e4m3.DECODE[e4m3.quantize(vn[0][b, g], s)] * np.float64(s)
            else:
                v = e4m3.bf16_bits_to_f64(vn[0][b, g])
            for h in range(g * group, (g + 1) * group):
                np.testing.assert_allclose(outs[0][b, h], v, rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_step_one_token_request_returns_its_own_value(cache):
    rng = np.random.default_rng(43)
    st, q, kn, vn = step_state(rng, [1, 1], hq=6, hkv=3, d=16, layers=2, cache=cache,
                               pool_pages=8)
    ab, outs = paged.decode_step(st, q, kn, vn, 0.25, cache=cache)
    for layer in range(2):
        for b in range(2):
            for h in range(6):
                g = h // 2
                if cache == "fp8":
                    s = np.float32(st["v_scale"][layer][g])
                    v = e4m3.DECODE[e4m3.quantize(vn[layer][b, g], s)] * np.float64(s)
                else:
                    v = e4m3.bf16_bits_to_f64(vn[layer][b, g])
                assert np.array_equal(outs[layer][b, h], v)


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_step_stale_request_is_neither_written_nor_read(cache):
    rng = np.random.default_rng(44)
    lens = [50, 23, 70, 9]
    st, q, kn, vn = step_state(rng, lens, layers=3, cache=cache, pool_pages=20)
    good = copy_state(st)
    st["pool_tags"][st["block_table"][2, 4]] += np.uint32(1)     # page reallocated
    good["expected_tags"][2, 4] = st["pool_tags"][st["block_table"][2, 4]]
    good["pool_tags"] = st["pool_tags"].copy()
    before = copy_state(st)
    ab, outs = paged.decode_step(st, q, kn, vn, 0.3, cache=cache)
    ab_good, outs_good = paged.decode_step(good, q, kn, vn, 0.3, cache=cache)
    assert ab.tolist() == [0, 0, 1, 0] and not ab_good.any()
    pages2 = set(st["block_table"][2, :5].tolist())
    for layer in range(3):
        for key in ("k_pool", "v_pool"):
            # request 2's pages keep every byte; the other requests' new rows
            # are exactly those of the run where request 2 was valid
            for p in pages2:
                assert np.array_equal(st[key][layer][p], before[key][layer][p])
            others = [p for p in range(20) if p not in pages2]
            assert np.array_equal(st[key][layer][others], good[key][layer][others])
        assert np.all(outs[layer][2] == 0.0)
        keep = [0, 1, 3]
        assert np.array_equal(outs[layer][keep], outs_good[layer][keep])
        assert np.any(outs_good[layer][2] != 0.0)


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_step_noop_tracker_writes_and_reads_the_stale_request(cache):
    rng = np.random.default_rng(45)
    lens = [50, 23, 70, 9]
    st, q, kn, vn = step_state(rng, lens, layers=2, cache=cache, pool_pages=20)
    good = copy_state(st)
    st["expected_tags"][2, 0] ^= np.uint32(5)                     # stale, but unchecked
    ab, outs = paged.decode_step(st, q, kn, vn, 0.3, cache=cache, verify=False)
    ab_good, outs_good = paged.decode_step(good, q, kn, vn, 0.3, cache=cache, verify=True)
    assert not ab.any() and not ab_good.any()
    for layer in range(2):
        assert np.array_equal(outs[layer], outs_good[layer])
        assert np.array_equal(st["k_pool"][layer], good["k_pool"][layer])
        assert np.array_equal(st["v_pool"][layer], good["v_pool"][layer])
    # the stale request's new row is there
    t = lens[2] - 1
    page, slot = int(st["block_table"][2, t // P]), t % P
    if cache == "fp8":
        want = e4m3.quantize(kn[0][2], st["k_scale"][0][:, None])
    else:
        want = kn[0][2]
    assert np.array_equal(st["k_pool"][0][page, :, slot], want)


def test_step_layers_are_independent():
    """Each layer appends into and reads from its own pools with its own
    scales: a three-layer step equals three one-layer steps."""
    rng = np.random.default_rng(46)
    st, q, kn, vn = step_state(rng, [30, 7, 48], layers=3, pool_pages=12)
    whole = copy_state(st)
    ab, outs = paged.decode_step(whole, q, kn, vn, 0.4)
    for layer in range(3):
        one = copy_state(st)
        for key in ("k_pool", "v_pool", "k_scale", "v_scale"):
            one[key] = [one[key][layer]]
        ab1, out1 = paged.decode_step(one, [q[layer]], [kn[layer]], [vn[layer]], 0.4)
        assert np.array_equal(ab1, ab)
        assert np.array_equal(out1[0], outs[layer])
        assert np.array_equal(one["k_pool"][0], whole["k_pool"][layer])
        assert np.array_equal(one["v_pool"][0], whole["v_pool"][layer])
