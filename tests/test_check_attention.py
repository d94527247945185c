"""Self-test of the attention tolerance gate (CPU only).

The gate must see an error confined to one (request, KV head) group, such as
one dropped or misplaced token, at the context lengths the workloads use.
Simulated outputs: the oracle's attention of a batch shaped like the mixed
8-request workload (64 query / 8 KV heads, lengths up to 8,192), and the same
attention with one token left out of one group only.
"""

import numpy as np
import pytest

from oracle import paged
from tests import helpers

HQ, HKV, D = 64, 8, 128
G = HQ // HKV


def _batch(rng, lens):
    q = rng.standard_normal((len(lens), HQ, D)).astype(np.float32)
    qb = (q.view(np.uint32) >> 16).astype(np.uint16)       # bf16 bits (truncated draws)
    K = [rng.standard_normal((HKV, L, D)) for L in lens]
    V = [0.5 * rng.standard_normal((HKV, L, D)) for L in lens]
    return qb, K, V


def _attend(qb, K, V, sm):
    return np.stack([paged.attend_request(qb[b], K[b], V[b], sm) for b in range(len(K))])


@pytest.mark.parametrize("drop", ["first", "middle", "last"])
def test_one_dropped_token_in_one_group_fails_the_gate(drop):
    rng = np.random.default_rng(77)
    lens = [8192, 1500, 3000, 6000, 1024, 2048, 5000, 7000]
    qb, K, V = _batch(rng, lens)
    sm = 1 / np.sqrt(D)
    want = _attend(qb, K, V, sm)
    b, g = 0, 3
    t = {"first": 0, "middle": 4097, "last": lens[0] - 1}[drop]
    keep = np.ones(lens[b], bool)
    keep[t] = False
    got = want.copy()
    got[b, g * G:(g + 1) * G] = paged.attend_request(
        qb[b, g * G:(g + 1) * G], K[b][g:g + 1, keep], V[b][g:g + 1, keep], sm)
    rel, mx, glob = helpers.attention_errors(got, want)
    # diluted over the whole batch the error would pass a global gate ...
    assert glob < helpers.REL_L2_TOL and mx.max() < helpers.MAX_ABS_TOL
    # ... but not the per-row one
    assert rel[b, g * G:(g + 1) * G].max() > 2 * helpers.REL_L2_TOL
    with pytest.raises(AssertionError, match="rows out of tolerance"):
        helpers.check_attention(got, want, label="dropped token")


def test_rounding_sized_noise_passes_and_zero_rows_are_enforced():
    rng = np.random.default_rng(78)
    lens = [2048, 17, 1, 600]
    qb, K, V = _batch(rng, lens)
    want = _attend(qb, K, V, 1 / np.sqrt(D))
    # relative noise of 2^-11 per element (f16 rounding of the probabilities)
    got = want * (1 + rng.uniform(-2.0 ** -11, 2.0 ** -11, want.shape))
    rel, mx = helpers.check_attention(got, want, label="noise")
    assert rel < helpers.REL_L2_TOL and mx < helpers.MAX_ABS_TOL
    got[1] = 0.0
    helpers.check_attention(got, want, zero_rows=[1], label="zero row")
    got[1, 5, 7] = 1e-30
    with pytest.raises(AssertionError, match="must be all zeros"):
        helpers.check_attention(got, want, zero_rows=[1], label="zero row")


def test_a_wrong_head_alone_fails_the_gate():
    """Two query heads of one request swapped: every other row is exact."""
    rng = np.random.default_rng(79)
    lens = [4096, 4096]
    qb, K, V = _batch(rng, lens)
    want = _attend(qb, K, V, 1 / np.sqrt(D))
    got = want.copy()
    got[1, [9, 10]] = got[1, [10, 9]]
    with pytest.raises(AssertionError, match="worst request 1 head (9|10)"):
        helpers.check_attention(got, want, label="swapped heads")
