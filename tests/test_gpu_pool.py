"""The host page pool driving the device tag check: tables built from pool
allocations, churn through free / realloc, and kv_verify_tags on the GPU
against the oracle's check and the pool's own bookkeeping."""

import numpy as np
import pytest
import torch

from oracle import paged
from tests.gpu_harness import DEV, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kv():
    import fp8_e4m3_paged_amd as k
    k.load()
    return k


def test_pool_driven_churn_aborts_exactly_the_stale_requests(kv):
    rng = np.random.default_rng(17)
    B = 48
    lens = rng.integers(1, 4000, size=B).astype(np.int32)
    need = -(-lens // 16)
    pool = kv.PagePool(int(need.sum() * 5 // 4) + 8, seed=2024)
    stride = int(need.max()) + 1
    bt = np.full((B, stride), -1, np.int32)
    ex = np.zeros((B, stride), np.uint32)
    for b in range(B):
        p, t = pool.alloc(int(need[b]))
        bt[b, :need[b]], ex[b, :need[b]] = p, t

    def device_check():
        abort = torch.full((B,), 7, dtype=torch.uint8, device=DEV)
        kv.kv_verify_tags(torch.from_numpy(pool.tags().view(np.int32)).to(DEV),
                          torch.from_numpy(bt).to(DEV), torch.from_numpy(ex.view(np.int32)).to(DEV),
                          torch.from_numpy(lens).to(DEV), abort)
        torch.cuda.synchronize()
        return abort.cpu().numpy()

    ab = device_check()
    assert not ab.any()
    pool.record_check(ab)
    # churn: 10% of the allocated pages are freed and reallocated; their owners
    # take new pages and record the new tags, except two stale requests that
    # keep their old mappings
    stale = [5, 31]
    owned = [(b, j) for b in range(B) for j in range(need[b])]
    pick = set(rng.choice(len(owned), size=len(owned) // 10, replace=False).tolist())
    pick |= {owned.index((b, int(need[b]) // 2)) for b in stale}
    freed = [owned[i] for i in sorted(pick)]
    pool.free(np.array([bt[b, j] for b, j in freed], np.int32))
    p, t = pool.alloc(len(freed))
    for (b, j), page, tag in zip(freed, p, t):
        if b in stale:
            continue                              # the stale request does not learn of it
        bt[b, j], ex[b, j] = page, tag
    want = paged.verify_tags(pool.tags(), bt, ex, lens, 16)
    ab = device_check()
    assert np.array_equal(ab, want)
    assert sorted(np.flatnonzero(ab).tolist()) == stale
    pool.record_check(ab)
    s = pool.stats()
    assert (s["checks"], s["requests_checked"], s["requests_aborted"]) == (2, 2 * B, 2)
    say(f"pool churn: {len(freed)} pages reallocated, aborted {stale}, "
        f"mismatch rate {s['mismatch_rate']:.4f}")
