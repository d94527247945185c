"""A host model of how the persistent attention kernel splits its work.

Mirrors ``attn_wave_kernel`` and its launch in ``csrc/decode_attn.hip``: the
(request, KV head, page) units of the requests the kernel accepts, numbered
request by request, then KV head, then page, each (request, KV head) led by
PENALTY units that hold no page; workgroup j of the G that share them takes
units [j U / G, (j + 1) U / G) and streams them as pieces that end on
partition boundaries and hold at most RUN_PAGES pages. Each piece owns the
partial slot of every partition whose first page it streams, and the piece
that ends a (request, KV head) also owns the slot after its last partition;
it writes its partial into the first slot it owns and marks the others empty.

Used by the CPU test of the slot-ownership argument and by the GPU needle
tests, which place tokens at piece boundaries.
"""

from __future__ import annotations

from dataclasses import dataclass

PAGE = 16
PENALTY = 64           # kPiecePenalty
RUN_PAGES = 1024       # kCoopRunPages
WAVES = 4              # kWaves
NUM_CUS = 256          # kNumCUs
MAX_TOKENS = 2048      # kWaveModeMaxTokens
MAX_BATCH = 4096       # kWaveModeMaxBatch


@dataclass(frozen=True)
class Piece:
    wg: int            # workgroup
    b: int             # request
    g: int             # KV head
    k0: int            # first page (index within the request)
    k_end: int         # one past the last page
    dst: int           # slot the partial goes to
    empty: tuple       # slots marked empty


def request_ok(L, aborted, max_seq_len, bt_stride):
    return (not aborted) and 1 <= L <= max_seq_len and -(-L // PAGE) <= bt_stride


def uses_wave_kernel(batch, hkv, max_seq_len, part_tokens):
    parts = -(-max_seq_len // part_tokens) if max_seq_len > 0 else 1
    return (parts > 1 and part_tokens <= MAX_TOKENS and batch <= MAX_BATCH
            and batch * hkv * parts >= WAVES * NUM_CUS)


def launch_grid(batch, hkv, max_seq_len, part_tokens):
    parts = -(-max_seq_len // part_tokens)
    return min(2 * NUM_CUS, -(-(batch * hkv * parts) // WAVES))


def split(lens, hkv, part_tokens, max_seq_len, bt_stride, aborted=None, grid=None):
    """Every piece the kernel streams, in workgroup order."""
    batch = len(lens)
    aborted = aborted if aborted is not None else [False] * batch
    if grid is None:
        grid = launch_grid(batch, hkv, max_seq_len, part_tokens)
    ppp = part_tokens // PAGE
    pre = [0]
    for b in range(batch):
        ok = request_ok(lens[b], aborted[b], max_seq_len, bt_stride)
        pre.append(pre[-1] + ((-(-lens[b] // PAGE) + PENALTY) if ok else 0))
    n_units = pre[batch] * hkv
    n_groups = min(grid, max(1, n_units // ppp))
    pieces = []
    for blk in range(n_groups):
        it = n_units * blk // n_groups
        u_end = n_units * (blk + 1) // n_groups
        while it < u_end:
            lo, hi = 0, batch - 1                 # last b with pre[b] * hkv <= it
            while lo < hi:
                mid = (lo + hi + 1) // 2
                if pre[mid] * hkv <= it:
                    lo = mid
                else:
                    hi = mid - 1
            b = lo
            L = lens[b]
            npg_b = -(-L // PAGE)
            ext_b = npg_b + PENALTY
            local = it - pre[b] * hkv
            g, r = divmod(local, ext_b)
            if r < PENALTY:
                it += min(PENALTY - r, u_end - it)
                continue
            k0 = r - PENALTY
            cap = (k0 + RUN_PAGES) // ppp * ppp
            k_end = min(npg_b, cap, k0 + (u_end - it))
            it += k_end - k0
            first_own = -(-k0 // ppp)
            end_own = -(-k_end // ppp)
            np_b = -(-npg_b // ppp)
            dst = first_own if first_own < end_own else np_b
            empty = [s for s in range(first_own, end_own) if s != dst]
            if k_end == npg_b and dst != np_b:
                empty.append(np_b)
            pieces.append(Piece(blk, b, g, k0, k_end, dst, tuple(empty)))
    return pieces
