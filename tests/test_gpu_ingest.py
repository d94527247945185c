"""GPU parity of prefill ingest (kv_amax_accumulate, kv_scales_from_amax,
kv_ingest_prefill) against the oracle in oracle/ingest.py: scales and codes
bit for bit, whole pools compared through the documented tile layouts, and
decode attention over an ingested pool within the tolerance."""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import synth
from oracle import e4m3, ingest, paged
from synth.device import DeviceState, prompt_rows
from tests import helpers
from tests.gpu_harness import DEV, say

pytestmark = pytest.mark.gpu
P = 16


@pytest.fixture(scope="module")
def kv():
    import fp8_e4m3_paged_amd as k
    k.load()
    return k


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def _random_bf16(rng, shape, specials=True):
    x = rng.normal(0.0, 1.5, size=shape).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    if specials:
        flat = bits.reshape(-1)
        idx = rng.choice(flat.size, size=max(1, flat.size // 97), replace=False)
        flat[idx] = rng.choice(np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x7F7F, 0x8000, 0x0001],
                                        dtype=np.uint16), size=idx.size)
    return bits


def _amax_gpu(kv, bits, init=None):
    a = torch.zeros(bits.shape[1], dtype=torch.float32, device=DEV) if init is None else \
        torch.from_numpy(np.asarray(init, np.float32)).to(DEV)
    kv.kv_amax_accumulate(_dev(bits), a)
    torch.cuda.synchronize()
    return a.cpu().numpy()


def test_amax_every_bf16_pattern(kv):
    """All 65,536 patterns (NaN, Inf, subnormals, -0 included), as one head and
    spread over 8 heads: the maximum finite magnitude, bit for bit."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(512, 1, 128)
    got = _amax_gpu(kv, bits)
    assert got.view(np.uint32)[0] == ingest.amax_finite(bits).view(np.uint32)[0]
    perm = np.random.default_rng(1).permutation(65536).astype(np.uint16).reshape(64, 8, 128)
    assert np.array_equal(_amax_gpu(kv, perm).view(np.uint32),
                          ingest.amax_finite(perm).view(np.uint32))


@pytest.mark.parametrize("rows,hkv", [(1, 1), (3, 2), (1000, 8), (4097, 4), (100_000, 8)])
def test_amax_random_sizes_and_accumulation(kv, rows, hkv):
    rng = np.random.default_rng(rows + hkv)
    bits = _random_bf16(rng, (rows, hkv, 128))
    want = ingest.amax_finite(bits)
    assert np.array_equal(_amax_gpu(kv, bits).view(np.uint32), want.view(np.uint32))
    # two calls over a split of the rows accumulate to the same; a larger start survives
    if rows > 1:
        a = torch.zeros(hkv, dtype=torch.float32, device=DEV)
        kv.kv_amax_accumulate(_dev(bits[: rows // 3]), a)
        kv.kv_amax_accumulate(_dev(bits[rows // 3:]), a)
        torch.cuda.synchronize()
        assert np.array_equal(a.cpu().numpy().view(np.uint32), want.view(np.uint32))
    big = np.full(hkv, 1e30, np.float32)
    big[0] = 0.0
    got = _amax_gpu(kv, bits, init=big)
    assert np.array_equal(got.view(np.uint32), np.maximum(big, want).view(np.uint32))
    say(f"amax rows={rows} hkv={hkv}: bit-exact")


def test_scales_from_amax_bit_exact(kv):
    rng = np.random.default_rng(3)
    a16 = (rng.integers(0, 0x8000, size=3000).astype(np.uint32) << 16).view(np.float32)
    a32 = rng.integers(0, 0x80000000, size=3000).astype(np.uint32).view(np.float32)
    special = np.array([0.0, -0.0, np.nan, np.inf, -np.inf, -1.0, 448.0, 224.0,
                        448.0 * 2.0 ** -126, np.nextafter(np.float32(448.0 * 2.0 ** -126), 0),
                        2.0 ** -149, 3.3895313892515355e38], np.float32)
    amax = np.concatenate([a16, a32, special]).astype(np.float32)
    out = torch.empty(amax.size, dtype=torch.float32, device=DEV)
    kv.kv_scales_from_amax(torch.from_numpy(amax).to(DEV), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32),
                          ingest.scales_from_amax(amax).view(np.uint32))


def _ingest_case(rng, cache, hkv=8, pool_pages=None):
    lens = [37, 0, 16, 1, 17, 33, 250, 1000, 15, 100, 64, 300]
    need = [max(1, -(-L // P)) for L in lens]
    pool_pages = pool_pages or sum(need) + 20
    perm = rng.permutation(pool_pages).astype(np.int32)
    bt = np.full((len(lens), max(need) + 2), -1, np.int32)
    off = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[off:off + n]
        off += n
    starts = (np.concatenate([[0], np.cumsum(lens)[:-1]]) + 5).astype(np.int32)
    n_rows = int(starts[-1] + lens[-1]) + 3
    kr = _random_bf16(rng, (n_rows, hkv, 128))
    vr = _random_bf16(rng, (n_rows, hkv, 128))
    ks = ingest.scales_from_amax(ingest.amax_finite(kr))
    vs = ingest.scales_from_amax(ingest.amax_finite(vr))
    if cache == "fp8":
        kt = rng.integers(0, 256, (pool_pages, hkv, 2048)).astype(np.uint8)
        vt = rng.integers(0, 256, (pool_pages, hkv, 2048)).astype(np.uint8)
    else:
        kt = rng.integers(0, 65536, (pool_pages, hkv, 2048)).astype(np.uint16)
        vt = rng.integers(0, 65536, (pool_pages, hkv, 2048)).astype(np.uint16)
    return dict(lens=np.array(lens, np.int32), bt=bt, starts=starts, kr=kr, vr=vr, ks=ks, vs=vs,
                kt=kt, vt=vt)


def _run_ingest(kv, c, cache, lens=None, starts=None, bt=None, abort=None, max_seq_len=None):
    lens = c["lens"] if lens is None else np.asarray(lens, np.int32)
    starts = c["starts"] if starts is None else np.asarray(starts, np.int32)
    bt = c["bt"] if bt is None else bt
    kp, vp = _dev(c["kt"]), _dev(c["vt"])
    if cache == "fp8":
        kp, vp = kp.view(torch.uint8), vp.view(torch.uint8)
    msl = int(lens.max()) if max_seq_len is None else max_seq_len
    kv.kv_ingest_prefill(_dev(c["kr"]), _dev(c["vr"]), torch.from_numpy(starts).to(DEV),
                         torch.from_numpy(lens).to(DEV), torch.from_numpy(bt).to(DEV), kp, vp,
                         msl, torch.from_numpy(c["ks"]).to(DEV), torch.from_numpy(c["vs"]).to(DEV),
                         abort=None if abort is None else torch.from_numpy(abort).to(DEV),
                         cache_dtype=0 if cache == "fp8" else 1)
    torch.cuda.synchronize()
    kg, vg = kp.cpu().numpy(), vp.cpu().numpy()
    if cache == "bf16":
        kg, vg = kg.view(np.uint16), vg.view(np.uint16)
    else:
        kg, vg = kg.view(np.uint8), vg.view(np.uint8)
    return (helpers.tiles_to_logical(kg, "k", cache), helpers.tiles_to_logical(vg, "v", cache))


def _oracle_ingest(c, cache, lens=None, starts=None, bt=None, abort=None, max_seq_len=None):
    kl = helpers.tiles_to_logical(c["kt"], "k", cache).copy()
    vl = helpers.tiles_to_logical(c["vt"], "v", cache).copy()
    ingest.ingest(kl, vl, c["kr"], c["vr"], c["starts"] if starts is None else starts,
                  c["lens"] if lens is None else lens, c["bt"] if bt is None else bt, cache,
                  c["ks"], c["vs"], abort=abort, max_seq_len=max_seq_len)
    return kl, vl


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_ingest_whole_pool_bit_exact(kv, cache):
    """Ragged prompts (empty, 1 token, page boundaries, long) into a pool full
    of stale bytes: every byte of both pools equals the oracle's, so written
    tiles, zeroed tails and untouched pages are all checked."""
    c = _ingest_case(np.random.default_rng(21), cache)
    gk, gv = _run_ingest(kv, c, cache)
    wk, wv = _oracle_ingest(c, cache)
    assert np.array_equal(gk, wk), f"{cache} K pool"
    assert np.array_equal(gv, wv), f"{cache} V pool"
    say(f"ingest {cache}: {int(c['lens'].sum())} tokens, whole pools bit-exact")


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_ingest_loops_over_more_pages_than_workgroups(kv, cache):
    """max_seq_len = 131072 gives 12 x 8192 (request, page) items, more than
    the 65,536 workgroups one launch uses, so workgroups take several items
    (almost all past their prompt's end); the pools must be the same."""
    c = _ingest_case(np.random.default_rng(23), cache)
    gk, gv = _run_ingest(kv, c, cache, max_seq_len=131072)
    wk, wv = _oracle_ingest(c, cache, max_seq_len=131072)
    assert np.array_equal(gk, wk), f"{cache} K pool"
    assert np.array_equal(gv, wv), f"{cache} V pool"


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_ingest_refusals(kv, cache):
    """Aborted requests, an out-of-pool page (skipped alone), rows outside the
    inputs and lengths over max_seq_len or beyond the table row write nothing."""
    c = _ingest_case(np.random.default_rng(22), cache)
    bt = c["bt"].copy()
    bt[7, 20] = 10 ** 7                         # request 7 (1000 tokens): one bad page
    bt[9, 2] = -3                               # request 9 (100 tokens)
    abort = np.zeros(len(c["lens"]), np.uint8)
    abort[[2, 6]] = 1
    starts = c["starts"].copy()
    starts[11] = c["kr"].shape[0] - 299         # request 11 needs 300 rows: one past the end
    starts[4] = -1
    lens = c["lens"].copy()
    lens[0] = P * bt.shape[1] + 1               # more pages than its table row
    for msl in (None, 299):
        gk, gv = _run_ingest(kv, c, cache, lens=lens, starts=starts, bt=bt, abort=abort,
                             max_seq_len=msl or int(lens.max()))
        wk, wv = _oracle_ingest(c, cache, lens=lens, starts=starts, bt=bt, abort=abort,
                                max_seq_len=msl)
        assert np.array_equal(gk, wk) and np.array_equal(gv, wv), f"{cache} max_seq_len={msl}"


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_ingest_layer_then_decode_attention(kv, cache):
    """The whole handoff on a mixed-length batch (64 q / 8 KV heads): scales
    calibrated on the GPU equal the oracle's bit for bit, the ingested pool
    equals the oracle's, and decode attention over it is within tolerance."""
    wl = synth.mixed_8req(max_steps=1)
    st = DeviceState(wl, kv, cache=cache, device=DEV, layers=[0], fill=False,
                     scales={0: (np.ones(8, np.float32), np.ones(8, np.float32))})
    kr, start = prompt_rows(wl, 0, "k", DEV)
    vr, _ = prompt_rows(wl, 0, "v", DEV)
    lens0 = torch.from_numpy(wl.seq_lens0.astype(np.int32)).to(DEV)
    ks = torch.empty(wl.num_kv_heads, dtype=torch.float32, device=DEV)
    vs = torch.empty_like(ks)
    kv.ingest_layer(kr, vr, start, lens0, st.block_table, st.k_pool[0], st.v_pool[0],
                    wl.max_seq_len, ks, vs, cache_dtype=0 if cache == "fp8" else 1)
    torch.cuda.synchronize()
    krh = kr.cpu().numpy().view(np.uint16)
    vrh = vr.cpu().numpy().view(np.uint16)
    ks_o = ingest.scales_from_amax(ingest.amax_finite(krh))
    vs_o = ingest.scales_from_amax(ingest.amax_finite(vrh))
    if cache == "fp8":
        assert np.array_equal(ks.cpu().numpy().view(np.uint32), ks_o.view(np.uint32))
        assert np.array_equal(vs.cpu().numpy().view(np.uint32), vs_o.view(np.uint32))
    shape = (wl.num_pages, wl.num_kv_heads, P, wl.head_dim)
    dt = np.uint8 if cache == "fp8" else np.uint16
    kl, vl = np.zeros(shape, dt), np.zeros(shape, dt)
    kt = st.k_pool[0].cpu().numpy()
    vt = st.v_pool[0].cpu().numpy()
    if cache == "bf16":
        kt, vt = kt.view(np.uint16), vt.view(np.uint16)
    gk, gv = helpers.tiles_to_logical(kt, "k", cache), helpers.tiles_to_logical(vt, "v", cache)
    # compare only the pages the requests own (the rest of the pool is whatever was there)
    ingest.ingest(kl, vl, krh, vrh, start.cpu().numpy(), wl.seq_lens0, wl.block_table, cache,
                  ks_o, vs_o)
    for b in range(wl.batch):
        for j in range(-(-int(wl.seq_lens0[b]) // P)):
            p = int(wl.block_table[b, j])
            assert np.array_equal(gk[p], kl[p]) and np.array_equal(gv[p], vl[p]), (b, j)
    # attention over the ingested tokens (no append: L = the prompt length)
    q = torch.from_numpy(wl.q_bits(0, 0).view(np.int16)).to(DEV)
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=DEV)
    n = kv.paged_decode_attn_workspace_bytes(
        wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.max_seq_len, 0,
        cache_dtype=kv.KV_CACHE_FP8_E4M3 if cache == "fp8" else kv.KV_CACHE_BF16)
    ws = torch.zeros(max(n, 256), dtype=torch.uint8, device=DEV)
    kv.paged_decode_attn(q, st.k_pool[0], st.v_pool[0], ks if cache == "fp8" else None,
                         vs if cache == "fp8" else None, st.block_table, lens0, wl.max_seq_len,
                         out, 1.0 / np.sqrt(wl.head_dim), workspace=ws,
                         cache_dtype=0 if cache == "fp8" else 1)
    torch.cuda.synchronize()
    want = paged.decode_attn(wl.q_bits(0, 0), kl, vl, ks_o, vs_o, wl.block_table,
                             wl.seq_lens0.astype(np.int32), 1.0 / np.sqrt(wl.head_dim), cache)
    rel, mx = helpers.check_attention(out.cpu().numpy(), want, label=f"ingest+attn {cache}")
    say(f"ingest_layer {cache}: scales and pages bit-exact; attention rel_l2={rel:.2e} max={mx:.2e}")


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def test_ingest_full_size_headline_prompts(kv):
    """One layer of the headline batch's prompts (64 x 8192 + U[0,1000]
    tokens), calibrated on the GPU and ingested in one launch, checked whole:
    each head's K and V scale equals the oracle's scale of the amax over all
    of that head's seeded values, bit for bit, and every page of every
    request holds the oracle's codes of its tokens under those scales, with
    zeros past each prompt's end (one (request, head) per thread)."""
    wl = synth.batch64_ctx8k(max_steps=1)
    st = DeviceState(wl, kv, cache="fp8", device=DEV, layers=[0], fill=False,
                     scales={0: (np.ones(8, np.float32), np.ones(8, np.float32))})
    kr, start = prompt_rows(wl, 0, "k", DEV)
    vr, _ = prompt_rows(wl, 0, "v", DEV)
    lens0 = torch.from_numpy(wl.seq_lens0.astype(np.int32)).to(DEV)
    ks = torch.empty(wl.num_kv_heads, dtype=torch.float32, device=DEV)
    vs = torch.empty_like(ks)
    kv.ingest_layer(kr, vr, start, lens0, st.block_table, st.k_pool[0], st.v_pool[0],
                    wl.max_seq_len, ks, vs)
    torch.cuda.synchronize()
    ksh, vsh = ks.cpu().numpy(), vs.cpu().numpy()
    del kr, vr
    hkv = wl.num_kv_heads
    groups = [(b, g) for b in range(wl.batch) for g in range(hkv)]
    bits = {}

    def head_amax(bg):
        b, g = bg
        L = int(wl.seq_lens0[b])
        kb = wl.kv_bits_head(0, "k", b, g, 0, L)
        vb = wl.kv_bits_head(0, "v", b, g, 0, L)
        bits[bg] = (kb, vb)
        return ingest.amax_finite(kb[:, None, :])[0], ingest.amax_finite(vb[:, None, :])[0]

    with ThreadPoolExecutor(_threads()) as ex:
        am = dict(zip(groups, ex.map(head_amax, groups)))
    ka = np.array([max(am[(b, g)][0] for b in range(wl.batch)) for g in range(hkv)], np.float32)
    va = np.array([max(am[(b, g)][1] for b in range(wl.batch)) for g in range(hkv)], np.float32)
    ks_o, vs_o = ingest.scales_from_amax(ka), ingest.scales_from_amax(va)
    assert np.array_equal(ksh.view(np.uint32), ks_o.view(np.uint32)), (ksh, ks_o)
    assert np.array_equal(vsh.view(np.uint32), vs_o.view(np.uint32)), (vsh, vs_o)

    def tiles_threaded(pool, kind):
        out = np.empty(pool.shape[:-1] + (P, 128), pool.dtype)
        cuts = np.linspace(0, pool.shape[0], 65).astype(np.int64)

        def conv(i):
            out[cuts[i]:cuts[i + 1]] = helpers.tiles_to_logical(pool[cuts[i]:cuts[i + 1]], kind, "fp8")

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(conv, range(64)))
        return out

    kl = tiles_threaded(st.k_pool[0].cpu().numpy(), "k")
    vl = tiles_threaded(st.v_pool[0].cpu().numpy(), "v")

    def pages_ok(bg):
        b, g = bg
        L = int(wl.seq_lens0[b])
        n = -(-L // P)
        ids = wl.block_table[b, :n]
        for pool, bb, sc in ((kl, bits[bg][0], ks_o[g]), (vl, bits[bg][1], vs_o[g])):
            want = np.zeros((n * P, 128), np.uint8)
            want[:L] = e4m3.quantize(bb, sc)
            if not np.array_equal(pool[ids, g].reshape(-1, 128), want):
                return bg
        return None

    with threadpool_limits(1), ThreadPoolExecutor(_threads()) as ex:
        bad = [r for r in ex.map(pages_ok, groups) if r is not None]
    assert not bad, f"pages differ for (request, head) {bad[:8]}"
    say(f"full-size ingest: scales of all {hkv} heads and all {sum(-(-int(L) // P) for L in wl.seq_lens0)}"
        f" pages x {hkv} heads bit-exact")


def _trap_scales(rng, count=2):
    """Scales s = fp32(amax / 448) (amax a random bf16) with the positive bf16
    values x whose plain fp32 quotient x / s lands exactly on an e4m3
    midpoint although the exact one does not, so that rounding the fp32
    quotient gives the wrong code: a scan of every finite pattern."""
    from oracle import e4m3
    pos = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)
    x32 = e4m3.bf16_bits_to_f64(pos).astype(np.float32)
    found = []
    for abits in rng.integers(0x3D4C, 0x4248, size=64).astype(np.uint16):
        s = np.float32(e4m3.bf16_bits_to_f64(np.array([abits]))[0] / 448.0)
        with np.errstate(over="ignore"):
            naive = e4m3.encode((x32 / s).astype(np.float64))
        traps = pos[e4m3.quantize(pos, s) != naive]
        if traps.size:
            found.append((traps.size, s, traps))
    found.sort(key=lambda t: -t[0])
    assert len(found) >= count
    return [(s, traps) for _, s, traps in found[:count]]


def test_ingest_reciprocal_and_division_paths_bit_exact(kv):
    """The FP8 page writer encodes a (page, head) tile without a division
    when the head's scale lies in [2^-63, 2^63] and every value of the tile
    is at most 2^63 in magnitude, and by division otherwise. This case mixes
    both on purpose, and every byte of both pools must equal the oracle's:
    clean tiles; one NaN, one infinity and one finite 2^70 confined to single
    tiles; scales on and just past both ends of the range and FLT_MIN; and
    two heads full of values (and their one-ulp neighbours) for which a
    plain fp32 quotient rounds to the wrong code."""
    rng = np.random.default_rng(31)
    hkv = 8
    lens = np.array([48, 40, 33, 16, 64, 7], np.int32)
    need = -(-lens // P)
    pool_pages = int(need.sum()) + 6
    perm = rng.permutation(pool_pages).astype(np.int32)
    bt = np.full((lens.size, int(need.max()) + 1), -1, np.int32)
    off = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[off:off + n]
        off += n
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    n_rows = int(lens.sum())
    kr = _random_bf16(rng, (n_rows, hkv, 128), specials=False)
    vr = _random_bf16(rng, (n_rows, hkv, 128), specials=False)
    ks = ingest.scales_from_amax(ingest.amax_finite(kr))
    vs = ingest.scales_from_amax(ingest.amax_finite(vr))
    ks[0], ks[1], ks[7] = 2.0 ** -63, 2.0 ** -64, 2.0 ** 63
    vs[2], vs[6] = 2.0 ** 64, np.finfo(np.float32).tiny
    vs[4] = np.nextafter(np.float32(2.0 ** -63), np.float32(0))
    # midpoint traps in K head 4 and V head 3: trap values with random signs, their
    # neighbours one ulp either side, and plain values
    for (arr, sc, g), (s, traps) in zip(((kr, ks, 4), (vr, vs, 3)), _trap_scales(rng)):
        sc[g] = s
        t = rng.choice(traps, size=n_rows * 128).astype(np.int32)
        t += rng.choice(np.array([-1, 0, 0, 0, 1]), size=t.size)
        t |= rng.integers(0, 2, size=t.size) << 15
        plain = rng.random(t.size) < 0.25
        arr[:, g, :] = np.where(plain, arr[:, g, :].reshape(-1), t).astype(np.uint16).reshape(n_rows, 128)
    # tile-local specials: (request, page, head, which)
    for b, j, g, which, val in ((1, 1, 2, "k", 0x7FC0), (2, 0, 5, "v", 0x7F80),
                                (3, 0, 1, "k", 0x6280), (0, 2, 6, "v", 0xFFC1)):
        row = starts[b] + j * P + 3
        (kr if which == "k" else vr)[row, g, 17] = val
    kt = rng.integers(0, 256, (pool_pages, hkv, 2048)).astype(np.uint8)
    vt = rng.integers(0, 256, (pool_pages, hkv, 2048)).astype(np.uint8)
    c = dict(lens=lens, bt=bt, starts=starts, kr=kr, vr=vr, ks=ks.astype(np.float32),
             vs=vs.astype(np.float32), kt=kt, vt=vt)
    gk, gv = _run_ingest(kv, c, "fp8")
    wk, wv = _oracle_ingest(c, "fp8")
    for name, g_, w_ in (("K", gk, wk), ("V", gv, wv)):
        bad = np.argwhere(g_ != w_)
        assert bad.size == 0, f"{name}: {len(bad)} bytes differ, first at {bad[:3].tolist()}"
    # the trap heads do hold values where a plain fp32 quotient rounds wrongly
    from oracle import e4m3
    for arr, s in ((kr[:, 4, :], ks[4]), (vr[:, 3, :], vs[3])):
        naive = e4m3.encode((e4m3.bf16_bits_to_f64(arr).astype(np.float32) / s).astype(np.float64))
        assert np.count_nonzero(naive != e4m3.quantize(arr, s)) > 100
    say("ingest fp8: reciprocal and division paths, whole pools bit-exact")
