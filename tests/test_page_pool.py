"""The host page pool and tag tracker (include/kvpool.h), on the CPU.

Pinned against a plain Python model of the rules the header states (LIFO
free list, all-or-nothing alloc and free, tag + 1 on every free, counters),
driven by random operation sequences; against the oracle's tag check (a
request still holding a freed page must abort, and only such requests); and
for thread safety."""

import threading

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as hs

from oracle import paged

EXHAUSTED, STATE = -7, -8


@pytest.fixture(scope="module")
def kv():
    import fp8_e4m3_paged_amd as k
    k.load()
    return k


class Model:
    """The pool's stated behaviour, written out plainly."""

    def __init__(self, n, tags, tracked):
        self.free = list(range(n - 1, -1, -1))      # top of the stack = end of the list
        self.alloc_set = set()
        self.tags = [int(t) for t in tags]
        self.tracked = tracked
        self.allocated = self.freed = 0

    def alloc(self, n):
        if n > len(self.free):
            return EXHAUSTED, None
        out = [self.free.pop() for _ in range(n)]
        self.alloc_set.update(out)
        self.allocated += n
        return 0, out

    def free_pages(self, pages):
        if len(set(pages)) != len(pages) or any(p not in self.alloc_set for p in pages):
            return STATE
        for p in pages:
            self.alloc_set.remove(p)
            if self.tracked:
                self.tags[p] = (self.tags[p] + 1) & 0xFFFFFFFF
            self.free.append(p)
        self.freed += len(pages)
        return 0


ops = hs.lists(hs.tuples(hs.sampled_from(["alloc", "free", "bad_free"]),
                         hs.integers(0, 9), hs.integers(0, 10 ** 6)), max_size=40)


@settings(max_examples=60, deadline=None)
@given(seq=ops, tracked=hs.booleans(), num_pages=hs.integers(0, 24))
def test_pool_follows_its_stated_rules(kv, seq, tracked, num_pages):
    pool = kv.PagePool(num_pages, tracked=tracked, seed=num_pages)
    model = Model(num_pages, pool.tags(), tracked)
    if not tracked:
        assert not pool.tags().any()
    held = []                                           # pages currently allocated, in order
    for op, n, salt in seq:
        if op == "alloc":
            want_st, want = model.alloc(n)
            try:
                pages, tags = pool.alloc(n)
                st = 0
            except kv.KvError as e:
                st = e.status
            assert st == want_st
            if st == 0:
                assert pages.tolist() == want
                assert tags.tolist() == [model.tags[p] for p in want]
                held.extend(want)
        elif op == "free" and held:
            k = 1 + salt % len(held)
            chosen = [held[(salt + 7 * i) % len(held)] for i in range(k)]
            chosen = list(dict.fromkeys(chosen))
            assert model.free_pages(chosen) == 0
            pool.free(chosen)
            held = [p for p in held if p not in chosen]
        elif op == "bad_free":
            # a repeated id, an unallocated page or an id out of range: refused, nothing changes
            cand = [(held[0], held[0]) if held else (num_pages,), (num_pages + salt,), (-1,)]
            bad = list(cand[salt % 3])
            before = pool.tags().copy()
            with pytest.raises(kv.KvError) as ei:
                pool.free(bad)
            assert ei.value.status == STATE
            assert np.array_equal(pool.tags(), before)
        assert pool.tags().tolist() == model.tags
        s = pool.stats()
        assert s["free_pages"] == len(model.free) == num_pages - len(model.alloc_set)
        assert s["pages_allocated"] == model.allocated and s["pages_freed"] == model.freed


def test_stale_mappings_are_exactly_the_aborted_requests(kv):
    """Requests record (page, tag) at allocation; some pages are freed and
    handed to new requests; the oracle's tag check over the pool's tags then
    flags exactly the requests that still hold a freed page."""
    rng = np.random.default_rng(5)
    pool = kv.PagePool(400, seed=9)
    lens = rng.integers(1, 300, size=12)
    need = -(-lens // 16)
    stride = int(need.max()) + 1
    bt = np.full((12, stride), -1, np.int32)
    ex = np.zeros((12, stride), np.uint32)
    for b in range(12):
        pages, tags = pool.alloc(int(need[b]))
        bt[b, :need[b]], ex[b, :need[b]] = pages, tags
    stale = [2, 7, 10]
    for b in stale:                      # the request's last page is freed and reused
        pool.free(bt[b, need[b] - 1: need[b]])
    newcomer, _ = pool.alloc(len(stale))
    assert set(newcomer.tolist()) == {int(bt[b, need[b] - 1]) for b in stale}   # LIFO reuse
    ab = paged.verify_tags(pool.tags(), bt, ex, lens, 16)
    assert sorted(np.flatnonzero(ab).tolist()) == stale
    # the mismatch-rate counters
    pool.record_check(ab)
    pool.record_check(np.zeros(12, np.uint8))
    s = pool.stats()
    assert (s["checks"], s["requests_checked"], s["requests_aborted"]) == (2, 24, 3)
    assert s["mismatch_rate"] == pytest.approx(3 / 24)


def test_noop_tracker_keeps_no_tags_and_counts_nothing(kv):
    pool = kv.PagePool(50, tracked=False)
    pages, tags = pool.alloc(20)
    assert not tags.any()
    pool.free(pages[:10])
    pages2, tags2 = pool.alloc(15)
    assert not tags2.any() and not pool.tags().any()
    pool.record_check(np.array([1, 0, 1], np.uint8))
    s = pool.stats()
    assert s["checks"] == 0 and s["requests_checked"] == 0 and s["mismatch_rate"] == 0.0
    assert s["free_pages"] == 50 - 20 + 10 - 15


def test_alloc_is_all_or_nothing_and_arguments_are_checked(kv):
    pool = kv.PagePool(8)
    a, _ = pool.alloc(6)
    with pytest.raises(kv.KvError) as ei:
        pool.alloc(3)
    assert ei.value.status == EXHAUSTED
    assert pool.stats()["free_pages"] == 2
    with pytest.raises(kv.KvError):
        pool.alloc(-1)
    with pytest.raises(kv.KvError):
        kv.PagePool(-5)
    lib = kv.load()
    assert lib.kv_pool_alloc(None, 1, None, None) == -1
    assert lib.kv_pool_free(None, None, 1) == -1
    assert lib.kv_pool_record_check(pool._h, None, 3) == -1
    lib.kv_pool_destroy(None)                           # ignored


def test_concurrent_alloc_and_free_never_share_a_page(kv):
    pool = kv.PagePool(4096, seed=1)
    owned = [[] for _ in range(8)]
    errors = []

    def worker(i):
        rng = np.random.default_rng(i)
        try:
            for _ in range(300):
                if owned[i] and rng.random() < 0.45:
                    k = int(rng.integers(1, len(owned[i]) + 1))
                    pool.free(owned[i][:k])
                    owned[i] = owned[i][k:]
                else:
                    try:
                        p, _ = pool.alloc(int(rng.integers(1, 12)))
                        owned[i].extend(p.tolist())
                    except kv.KvError as e:
                        assert e.status == EXHAUSTED
        except Exception as e:                         # reported below
            errors.append(e)

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors
    flat = [p for o in owned for p in o]
    assert len(flat) == len(set(flat))
    s = pool.stats()
    assert s["free_pages"] == 4096 - len(flat)
    assert s["pages_allocated"] - s["pages_freed"] == len(flat)
