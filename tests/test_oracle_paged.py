"""Pins for the oracle's tag check, append and attention (CPU only).

Each test ties the oracle to something outside itself: a pure-Python brute
force written independently below, a closed form (one token, uniform V, zero
temperature, two tokens), an invariant (page permutation, untouched bytes),
or a behaviour the pages state (a stale tag aborts exactly its request; the
check covers the pages a request reads).
"""

import math

import numpy as np
import pytest

import synth
from oracle import e4m3, paged

P = 16


# ---------------------------------------------------------------------------
# small random paged state (oracle-only; values straight from numpy)
# ---------------------------------------------------------------------------
def small_state(rng, batch=3, hq=4, hkv=2, d=8, lens=(37, 16, 5), pool_pages=20,
                cache="fp8"):
    need = [-(-L // P) for L in lens]
    perm = rng.permutation(pool_pages)
    max_pages = max(need) + 1
    bt = np.full((batch, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        bt[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    if cache == "fp8":
        kp = rng.integers(0, 256, size=(pool_pages, hkv, P, d)).astype(np.uint8)
        vp = rng.integers(0, 256, size=(pool_pages, hkv, P, d)).astype(np.uint8)
        # keep NaN codes out of the attention inputs
        kp[(kp & 0x7F) == 0x7F] = 0x3C
        vp[(vp & 0x7F) == 0x7F] = 0x3C
    else:
        kp = synth._f32_to_bf16_bits(rng.normal(0, 1, (pool_pages, hkv, P, d)).astype(np.float32))
        vp = synth._f32_to_bf16_bits(rng.normal(0, 1, (pool_pages, hkv, P, d)).astype(np.float32))
    q = synth._f32_to_bf16_bits(rng.normal(0, 1, (batch, hq, d)).astype(np.float32))
    ks = np.float32(rng.uniform(0.001, 0.02, hkv)).astype(np.float32)
    vs = np.float32(rng.uniform(0.001, 0.02, hkv)).astype(np.float32)
    return dict(q=q, kp=kp, vp=vp, bt=bt, lens=np.array(lens, dtype=np.int32), ks=ks, vs=vs)


def brute_force_attention(st, sm_scale, cache="fp8"):
    """Pure-Python loops over (b, h, j, d): gather, dequantize, softmax, sum."""
    q, kp, vp, bt, lens = st["q"], st["kp"], st["vp"], st["bt"], st["lens"]
    batch, hq, d = q.shape
    hkv = kp.shape[1]
    out = [[[0.0] * d for _ in range(hq)] for _ in range(batch)]

    def bf(bits):
        return float(np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0])

    def dq(code, s):
        if cache == "fp8":
            code = int(code)
            sign = -1.0 if code & 0x80 else 1.0
            ex, man = (code >> 3) & 15, code & 7
            v = (man / 8.0) * 2.0 ** -6 if ex == 0 else (1 + man / 8.0) * 2.0 ** (ex - 7)
            return sign * v * float(s)
        return bf(code)

    for b in range(batch):
        L = int(lens[b])
        for h in range(hq):
            g = h // (hq // hkv)
            scores = []
            for t in range(L):
                page = int(bt[b][t // P])
                acc = 0.0
                for i in range(d):
                    acc += bf(q[b][h][i]) * dq(kp[page][g][t % P][i], st["ks"][g])
                scores.append(acc * sm_scale)
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            z = sum(w)
            for t in range(L):
                page = int(bt[b][t // P])
                for i in range(d):
                    out[b][h][i] += w[t] / z * dq(vp[page][g][t % P][i], st["vs"][g])
    return np.array(out)


def run_oracle(st, sm_scale, cache="fp8", abort=None):
    return paged.decode_attn(st["q"], st["kp"], st["vp"], st["ks"], st["vs"], st["bt"],
                             st["lens"], sm_scale, cache, abort)


@pytest.mark.parametrize("cache", ["fp8", "bf16"])
def test_attention_matches_pure_python_bruteforce(cache):
    rng = np.random.default_rng(3)
    st = small_state(rng, cache=cache)
    sm = 1 / math.sqrt(8)
    got = run_oracle(st, sm, cache)
    want = brute_force_attention(st, sm, cache)
    assert np.max(np.abs(got - want)) <= 1e-12


def test_single_token_returns_v():
    rng = np.random.default_rng(4)
    st = small_state(rng, lens=(1, 1, 1))
    out = run_oracle(st, 0.3)
    for b in range(3):
        page = st["bt"][b][0]
        for h in range(4):
            g = h // 2
            v0 = e4m3.DECODE[st["vp"][page][g][0]] * np.float64(st["vs"][g])
            assert np.array_equal(out[b][h], v0)


def test_uniform_v_returns_v():
    rng = np.random.default_rng(5)
    st = small_state(rng)
    st["vp"][:] = 0x44          # every V element is the same code
    out = run_oracle(st, 0.5)
    for h in range(4):
        g = h // 2
        np.testing.assert_allclose(out[:, h, :], e4m3.DECODE[0x44] * np.float64(st["vs"][g]),
                                   rtol=1e-14)


def _mean_v(st, b, g, L, cache="fp8"):
    V = paged.dequant_request(st["vp"], st["bt"][b], L, P, st["vs"], cache)
    return V[g].mean(axis=0)


def test_zero_temperature_gives_mean_of_v():
    rng = np.random.default_rng(6)
    st = small_state(rng)
    out = run_oracle(st, 0.0)
    for b, L in enumerate(st["lens"]):
        for h in range(4):
            np.testing.assert_allclose(out[b][h], _mean_v(st, b, h // 2, int(L)), rtol=1e-12,
                                       atol=1e-15)


def test_equal_keys_give_mean_of_v():
    rng = np.random.default_rng(7)
    st = small_state(rng)
    st["kp"][:] = 0x3A
    out = run_oracle(st, 0.7)
    for b, L in enumerate(st["lens"]):
        for h in range(4):
            np.testing.assert_allclose(out[b][h], _mean_v(st, b, h // 2, int(L)), rtol=1e-12,
                                       atol=1e-15)


def test_two_tokens_closed_form():
    rng = np.random.default_rng(8)
    st = small_state(rng, lens=(2, 2, 2))
    sm = 0.37
    out = run_oracle(st, sm)
    for b in range(3):
        page = st["bt"][b][0]
        for h in range(4):
            g = h // 2
            qv = e4m3.bf16_bits_to_f64(st["q"][b][h])
            k0 = e4m3.DECODE[st["kp"][page][g][0]] * np.float64(st["ks"][g])
            k1 = e4m3.DECODE[st["kp"][page][g][1]] * np.float64(st["ks"][g])
            v0 = e4m3.DECODE[st["vp"][page][g][0]] * np.float64(st["vs"][g])
            v1 = e4m3.DECODE[st["vp"][page][g][1]] * np.float64(st["vs"][g])
            w0 = 1.0 / (1.0 + math.exp((qv @ k1 - qv @ k0) * sm))   # logistic
            np.testing.assert_allclose(out[b][h], w0 * v0 + (1 - w0) * v1, rtol=1e-12,
                                       atol=1e-15)


def test_huge_scores_select_the_argmax_token():
    rng = np.random.default_rng(9)
    st = small_state(rng)
    out = run_oracle(st, 1e6)
    for b, L in enumerate(st["lens"]):
        K = paged.dequant_request(st["kp"], st["bt"][b], int(L), P, st["ks"], "fp8")
        V = paged.dequant_request(st["vp"], st["bt"][b], int(L), P, st["vs"], "fp8")
        for h in range(4):
            s = K[h // 2] @ e4m3.bf16_bits_to_f64(st["q"][b][h])
            top = np.flatnonzero(s == s.max())
            np.testing.assert_allclose(out[b][h], V[h // 2][top].mean(axis=0), rtol=1e-9)


def test_physical_page_permutation_is_invisible():
    rng = np.random.default_rng(10)
    st = small_state(rng)
    out = run_oracle(st, 0.4)
    perm = rng.permutation(st["kp"].shape[0])
    inv = np.argsort(perm)
    st2 = dict(st)
    st2["kp"] = st["kp"][perm]           # new page i holds old page perm[i]
    st2["vp"] = st["vp"][perm]
    bt2 = st["bt"].copy()
    m = bt2 >= 0
    bt2[m] = inv[bt2[m]]
    st2["bt"] = bt2
    assert np.array_equal(run_oracle(st2, 0.4), out)


def test_mha_is_gqa_with_group_one():
    rng = np.random.default_rng(12)
    st = small_state(rng, hq=2, hkv=2)
    out = run_oracle(st, 0.3)
    for g in range(2):
        sub = dict(st)
        sub["q"] = st["q"][:, g:g + 1]
        sub["kp"] = st["kp"][:, g:g + 1]
        sub["vp"] = st["vp"][:, g:g + 1]
        sub["ks"] = st["ks"][g:g + 1]
        sub["vs"] = st["vs"][g:g + 1]
        np.testing.assert_array_equal(run_oracle(sub, 0.3)[:, 0], out[:, g])


def test_aborted_empty_and_unmapped_requests_output_zero():
    rng = np.random.default_rng(13)
    st = small_state(rng)
    abort = np.array([0, 1, 0], dtype=np.uint8)
    st["lens"] = np.array([37, 16, 0], dtype=np.int32)
    out = run_oracle(st, 0.3, abort=abort)
    assert np.all(out[1] == 0) and np.all(out[2] == 0) and np.any(out[0] != 0)
    st["lens"] = np.array([37, 16, 5], dtype=np.int32)
    st["bt"][0][1] = 10 ** 6
    out = run_oracle(st, 0.3)
    assert np.all(out[0] == 0) and np.any(out[1] != 0)


# ---------------------------------------------------------------------------
# tag check
# ---------------------------------------------------------------------------
def test_verify_all_matching_is_all_zero():
    for make in (synth.tiny_1req, synth.uniform_32req, synth.batch64_ctx8k):
        wl = make()
        ab = paged.verify_tags(wl.pool_tags, wl.block_table, wl.expected_tags,
                               wl.seq_lens_at(0), P)
        assert ab.dtype == np.uint8 and not ab.any()


def test_verify_flags_exactly_the_stale_request_and_ignores_the_tail():
    wl = synth.mixed_8req()
    ab = paged.verify_tags(wl.pool_tags, wl.block_table, wl.expected_tags,
                           wl.seq_lens_at(0), P)
    assert np.flatnonzero(ab).tolist() == list(wl.stale)
    # the generator fills entries past each request's pages with garbage ids
    # and tags; a tag check that looked at them would abort everything
    assert (wl.block_table < 0).any() or (wl.block_table >= wl.num_pages).any()


def test_verify_page_boundaries_and_bad_ids():
    rng = np.random.default_rng(14)
    tags = rng.integers(0, 2 ** 32, 50, dtype=np.uint64).astype(np.uint32)
    bt = np.array([[3, 7, 9], [4, -1, 77]], dtype=np.int32)
    exp = np.zeros_like(bt, dtype=np.uint32)
    for b in range(2):
        for j in range(3):
            if 0 <= bt[b, j] < 50:
                exp[b, j] = tags[bt[b, j]]
    v = lambda lens: paged.verify_tags(tags, bt, exp, np.array(lens), P).tolist()  # noqa
    assert v([48, 16]) == [0, 0]          # request 1 only reads page 0
    assert v([48, 17]) == [0, 1]          # token 16 lives on the bad page -1
    assert v([49, 0]) == [1, 0]           # 49 tokens need a 4th page the row lacks
    assert v([-1, 1]) == [1, 0]           # a negative length is invalid
    exp2 = exp.copy()
    exp2[0, 2] ^= 0x80000000
    assert paged.verify_tags(tags, bt, exp2, np.array([32, 1]), P).tolist() == [0, 0]
    assert paged.verify_tags(tags, bt, exp2, np.array([33, 1]), P).tolist() == [1, 0]


def test_churn_aborts_exactly_the_two_stale_requests():
    wl = synth.skewed_16req()
    ab0 = paged.verify_tags(wl.pool_tags, wl.block_table, wl.expected_tags,
                            wl.seq_lens_at(0), P)
    assert not ab0.any()
    stale = wl.notes["churn_stale"]
    bumped = wl.apply_churn(np.random.default_rng(wl.notes["churn_rng_seed"]), 0.10, stale)
    allocated = int(wl.pages_allocated.sum())
    assert abs(len(bumped) - 0.10 * allocated) <= len(stale) + 1
    ab1 = paged.verify_tags(wl.pool_tags, wl.block_table, wl.expected_tags,
                            wl.seq_lens_at(1), P)
    assert sorted(np.flatnonzero(ab1).tolist()) == sorted(stale)


# ---------------------------------------------------------------------------
# append
# ---------------------------------------------------------------------------
def test_append_writes_only_the_target_rows():
    rng = np.random.default_rng(15)
    st = small_state(rng)
    kp0, vp0 = st["kp"].copy(), st["vp"].copy()
    k_new = synth._f32_to_bf16_bits(rng.normal(0, 0.02, (3, 2, 8)).astype(np.float32))
    v_new = synth._f32_to_bf16_bits(rng.normal(0, 0.02, (3, 2, 8)).astype(np.float32))
    pos = st["lens"] - 1
    abort = np.array([0, 0, 1], dtype=np.uint8)
    paged.append_fp8(st["kp"], st["vp"], k_new, v_new, np.arange(3), pos, st["bt"],
                     st["ks"], st["vs"], abort)
    changed = np.argwhere((st["kp"] != kp0).any(axis=(1, 3)) | (st["vp"] != vp0).any(axis=(1, 3)))
    allowed = {(int(st["bt"][b][pos[b] // P]), int(pos[b] % P)) for b in (0, 1)}
    for page, slot in changed:
        assert (int(page), int(slot)) in allowed
    for b in (0, 1):
        page, slot = int(st["bt"][b][pos[b] // P]), int(pos[b] % P)
        for g in range(2):
            x = e4m3.bf16_bits_to_f64(k_new[b][g]) / np.float64(st["ks"][g])
            codes = st["kp"][page][g][slot]
            # each code is a nearest representable value of x / s
            err = np.abs(e4m3.DECODE[codes] - x)
            alt = np.abs(e4m3.DECODE[:0x7F][None, :] - np.abs(x)[:, None]).min(axis=1)
            assert np.all(err <= alt + 0.0)
    # the aborted request's target row is untouched
    page, slot = int(st["bt"][2][pos[2] // P]), int(pos[2] % P)
    assert np.array_equal(st["kp"][page, :, slot], kp0[page, :, slot])


def test_append_skips_unmapped_targets():
    rng = np.random.default_rng(16)
    st = small_state(rng)
    kp0 = st["kp"].copy()
    k_new = np.zeros((2, 2, 8), dtype=np.uint16)
    paged.append_fp8(st["kp"], st["vp"], k_new, k_new, np.array([0, 5]),
                     np.array([16 * 3 + 1, 0]), st["bt"], st["ks"], st["vs"])
    assert np.array_equal(st["kp"], kp0)     # page slot 3 of request 0 is -1; request 5 absent
