"""The persistent attention kernel's work split, checked on the host model
(tests/wave_split_model.py) over random shapes: every page of every accepted
(request, KV head) is streamed by exactly one piece, and every partial slot
the cross-partition reduction reads is written exactly once (by the partial
of the piece that owns it, or as an empty mark). Requests the kernel refuses
get no piece at all."""

import numpy as np
import pytest

import synth
from tests import wave_split_model as ws


def _check(lens, hkv, pt, msl, stride, aborted, grid=None):
    pieces = ws.split(lens, hkv, pt, msl, stride, aborted, grid)
    ppp = pt // ws.PAGE
    pages, slots = {}, {}
    for pc in pieces:
        assert 1 <= pc.k_end - pc.k0 <= ws.RUN_PAGES
        # a piece ends on a partition boundary, at the end of its request,
        # or where its workgroup's share ends
        for k in range(pc.k0, pc.k_end):
            key = (pc.b, pc.g, k)
            assert key not in pages, f"page {key} streamed twice"
            pages[key] = pc.wg
        for s in (pc.dst,) + pc.empty:
            key = (pc.b, pc.g, s)
            assert key not in slots, f"slot {key} written twice"
            slots[key] = pc.wg
    for b, L in enumerate(lens):
        ok = ws.request_ok(L, aborted[b], msl, stride)
        npg = -(-L // ws.PAGE)
        n_slots = -(-npg // ppp) + 1          # the partitions and the extra slot
        for g in range(hkv):
            got_pages = sum((b, g, k) in pages for k in range(max(npg, 0)))
            got_slots = sum((b, g, s) in slots for s in range(max(n_slots, 0)))
            if ok:
                assert got_pages == npg, (b, g, got_pages, npg)
                assert got_slots == n_slots, (b, g, got_slots, n_slots)
            else:
                assert got_pages == 0 and got_slots == 0
    return pieces


def test_random_shapes():
    rng = np.random.default_rng(2026)
    n_partial_starts = 0
    for trial in range(400):
        batch = int(rng.integers(1, 160))
        hkv = int(rng.choice([1, 2, 4, 8]))
        pt = 16 * int(rng.integers(1, ws.MAX_TOKENS // 16 + 1))
        top = int(rng.choice([200, 3000, 40_000]))
        lens = rng.integers(0, top, batch).tolist()
        if trial % 3 == 0:
            lens[int(rng.integers(batch))] = top
        msl = max(max(lens), 1)
        stride = -(-msl // 16) + int(rng.integers(0, 2))
        aborted = (rng.random(batch) < 0.1).tolist()
        if rng.random() < 0.2:                     # a few too long for the row / the maximum
            lens[int(rng.integers(batch))] = msl + 16
        grid = None if rng.random() < 0.7 else int(rng.integers(1, 600))
        pieces = _check(lens, hkv, pt, msl, stride, aborted, grid)
        ppp = pt // 16
        n_partial_starts += sum(pc.k0 % ppp != 0 for pc in pieces)
    assert n_partial_starts > 100     # shares that start inside partitions were exercised


def test_skewed_workload_pieces():
    """The skewed 16-request workload (lengths to 131,072, 512-token
    partitions): the launch the benchmark times."""
    wl = synth.skewed_16req(max_steps=2)
    for step in (0, 1):
        lens = wl.seq_lens_at(step).tolist()
        assert ws.uses_wave_kernel(wl.batch, wl.num_kv_heads, wl.max_seq_len, 512)
        pieces = _check(lens, wl.num_kv_heads, 512, wl.max_seq_len, wl.block_table.shape[1],
                        [False] * wl.batch)
        assert len({pc.wg for pc in pieces}) == ws.launch_grid(wl.batch, wl.num_kv_heads,
                                                               wl.max_seq_len, 512)


@pytest.mark.parametrize("lens", [[1], [16, 17, 0, 5000], [131072, 512, 512]])
def test_small_cases(lens):
    _check(lens, 8, 16, max(lens), -(-max(lens) // 16), [False] * len(lens))
    _check(lens, 1, 2048, max(lens), -(-max(lens) // 16), [False] * len(lens), grid=3)
