"""Seeded synthetic inputs for the paged FP8 KV-cache decode step.

This module is shared by the oracle side and the GPU side of every test and of
the benchmark. It holds no arithmetic of the method: no E4M3 coding, no tag
check and no attention. It only defines *which* values, lengths, page
assignments and tags a workload has.

Values. Every bf16 input value is a pure function of (seed, tensor, layer,
request, token, head, dim): a counter-based hash (two rounds of the
MurmurHash3 32-bit finaliser, ``fmix32``) picks one of 65536 entries of a
table of standard-normal quantiles, ``Phi^-1((i + 0.5) / 65536)`` rounded to
bfloat16, times sigma (1 or 0.5, exact in bf16). So the values are bf16
draws from N(0, sigma^2) truncated at +-4.33 sigma, and any single request
can be regenerated alone. ``synth.device`` evaluates the same integer hash
with torch on the GPU and gets the same bits; that is how multi-GB pools are
made on the device while the oracle regenerates one request on the host.

Structure (lengths, page permutation, tags, which request is stale) comes
from ``numpy.random.Generator(PCG64(1000 + config_index))``.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from statistics import NormalDist

import numpy as np

M32 = 0xFFFFFFFF
_C1 = 0x85EBCA6B
_C2 = 0xC2B2AE35


# --------------------------------------------------------------------------
# counter-based hash (numpy uint32)
# --------------------------------------------------------------------------
def fmix32(h):
    """MurmurHash3's 32-bit finaliser; numpy uint32 products wrap mod 2^32."""
    h = np.asarray(h, dtype=np.uint32)
    h = h ^ (h >> np.uint32(16))
    h = h * np.uint32(_C1)
    h = h ^ (h >> np.uint32(13))
    h = h * np.uint32(_C2)
    h = h ^ (h >> np.uint32(16))
    return h


def _fmix32_int(x: int) -> int:
    return int(fmix32(np.array([x & M32], dtype=np.uint32))[0])


def stream_key(seed: int, *parts: int) -> tuple[int, int]:
    """Two 32-bit keys identifying one tensor stream (seed, tensor id, ...)."""
    h = _fmix32_int(seed)
    for p in parts:
        h = _fmix32_int(h ^ ((p + 0x9E3779B9) & M32))
    return h, _fmix32_int(h ^ 0x5BD1E995)


def table_index(key: tuple[int, int], ctr) -> np.ndarray:
    """16-bit table index for each counter value (counters < 2^32)."""
    k1, k2 = key
    h = fmix32(np.asarray(ctr, dtype=np.uint32) ^ np.uint32(k1))
    h = fmix32(h + np.uint32(k2))
    return (h >> np.uint32(16)).astype(np.int64)


# --------------------------------------------------------------------------
# bf16 normal quantile tables
# --------------------------------------------------------------------------
def _f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest even (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def _make_table(sigma: float) -> np.ndarray:
    nd = NormalDist()
    q = np.array([nd.inv_cdf((i + 0.5) / 65536.0) for i in range(65536)])
    return _f32_to_bf16_bits((q * sigma).astype(np.float32))


_TABLES: dict[float, np.ndarray] = {}


def normal_table(sigma: float) -> np.ndarray:
    """uint16[65536] bf16 bits of sigma * Phi^-1((i + 0.5) / 65536)."""
    if sigma not in _TABLES:
        if sigma == 1.0:
            _TABLES[sigma] = _make_table(1.0)
        else:
            # sigma * bf16(q) computed exactly for power-of-two sigma
            base = normal_table(1.0).astype(np.uint32) << np.uint32(16)
            _TABLES[sigma] = _f32_to_bf16_bits(base.view(np.float32) * np.float32(sigma))
    return _TABLES[sigma]


def normal_bf16(key, ctr, sigma: float) -> np.ndarray:
    """bf16 bits of N(0, sigma^2) draws at the given counters."""
    return normal_table(sigma)[table_index(key, ctr)]


# tensor ids inside a workload's key space
T_K, T_V, T_Q = 1, 2, 3


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclass
class Workload:
    """One synthetic decode workload: shapes, page tables, tags and values.

    ``seq_lens0[b]`` tokens of request b are in the pool before the first
    step; step s appends token ``seq_lens0[b] + s`` and attends over
    ``seq_lens0[b] + s + 1`` tokens.
    """

    name: str
    seed: int
    batch: int
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    seq_lens0: np.ndarray
    block_table: np.ndarray
    pool_tags: np.ndarray
    expected_tags: np.ndarray
    num_pages: int
    k_sigma: float
    v_sigma: float
    q_sigma: float
    max_steps: int
    stale: tuple = ()
    partition_tokens: int = 0
    notes: dict = field(default_factory=dict)

    # ---- lengths ---------------------------------------------------------
    def seq_lens_at(self, step: int) -> np.ndarray:
        """Attention span of each request at step s (appended token included)."""
        return (self.seq_lens0 + step + 1).astype(np.int32)

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens0.max()) + self.max_steps

    # ---- values ----------------------------------------------------------
    def _kv_key(self, layer: int, kind: str, b: int):
        tid = T_K if kind == "k" else T_V
        return stream_key(self.seed, tid, layer, b)

    def kv_sigma(self, kind: str) -> float:
        return self.k_sigma if kind == "k" else self.v_sigma

    def kv_bits(self, layer: int, kind: str, b: int, t0: int, t1: int) -> np.ndarray:
        """bf16 bits [t1 - t0][Hkv][D] of tokens t0..t1-1 of request b.

        Counter of (t, g, d) = (t * Hkv + g) * D + d, evaluated head by head."""
        return np.stack([self.kv_bits_head(layer, kind, b, g, t0, t1)
                         for g in range(self.num_kv_heads)], axis=1)

    def kv_bits_head(self, layer: int, kind: str, b: int, g: int, t0: int, t1: int) -> np.ndarray:
        """bf16 bits [t1 - t0][D] of KV head g only (the same values as kv_bits)."""
        hkv, d = self.num_kv_heads, self.head_dim
        t = np.arange(t0, t1, dtype=np.uint32)[:, None]
        j = np.arange(d, dtype=np.uint32)[None, :]
        ctr = (t * np.uint32(hkv) + np.uint32(g)) * np.uint32(d) + j
        return normal_bf16(self._kv_key(layer, kind, b), ctr, self.kv_sigma(kind))

    def new_token_bits(self, layer: int, kind: str, step: int) -> np.ndarray:
        """bf16 bits [B][Hkv][D] of the token each request appends at step s."""
        return np.stack([
            self.kv_bits(layer, kind, b, int(self.seq_lens0[b]) + step,
                         int(self.seq_lens0[b]) + step + 1)[0]
            for b in range(self.batch)
        ])

    def q_bits(self, layer: int, step: int) -> np.ndarray:
        """bf16 bits [B][Hq][D] of the decode queries of one layer and step."""
        hq, d = self.num_q_heads, self.head_dim
        ctr = np.arange(self.batch * hq * d, dtype=np.uint32).reshape(self.batch, hq, d)
        return normal_bf16(stream_key(self.seed, T_Q, layer, step), ctr, self.q_sigma)

    def initial_scales(self, layer: int) -> tuple[np.ndarray, np.ndarray]:
        """fp32 (k_scale, v_scale) per KV head = amax / 448 over the initial pool.

        amax is the largest |value| of that (layer, head) over every request's
        initial tokens; a zero amax gives scale 1.0. Host evaluation: use only
        for workloads small enough to regenerate on the CPU.
        """
        out = []
        for kind in ("k", "v"):
            amax = np.zeros(self.num_kv_heads, dtype=np.float32)
            for b in range(self.batch):
                bits = self.kv_bits(layer, kind, b, 0, int(self.seq_lens0[b]))
                vals = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
                if vals.size:
                    amax = np.maximum(amax, np.abs(vals).max(axis=(0, 2)))
            out.append(scales_from_amax(amax))
        return out[0], out[1]

    # ---- tags ------------------------------------------------------------
    def pages_of(self, b: int, step: int = 0) -> int:
        return -(-int(self.seq_lens_at(step)[b]) // self.page_size)

    def apply_churn(self, rng: np.random.Generator, fraction: float = 0.10,
                    stale: tuple = ()) -> np.ndarray:
        """Free and reallocate ``fraction`` of the allocated pages with a tag bump.

        Each chosen page keeps its owner; its pool tag is incremented (mod
        2^32) and the owner's expected tag follows, except for the requests in
        ``stale``, which keep their old (now stale) expectation. At least one
        page inside the current span of each stale request is chosen. Returns
        the physical ids that were bumped.
        """
        owners = []
        for b in range(self.batch):
            for j in range(self.block_table.shape[1]):
                p = int(self.block_table[b, j])
                if 0 <= p < self.num_pages and j < self.pages_allocated[b]:
                    owners.append((p, b, j))
        owners = np.array(owners, dtype=np.int64)
        n = max(1, int(round(fraction * len(owners))))
        pick = set(rng.choice(len(owners), size=n, replace=False).tolist())
        for sb in stale:
            span = self.pages_of(sb, self.notes.get("churn_step", 0))
            cand = [i for i, (p, b, j) in enumerate(owners) if b == sb and j < span]
            if not any(i in pick for i in cand):
                pick.add(int(rng.choice(cand)))
        bumped = []
        for i in sorted(pick):
            p, b, j = (int(x) for x in owners[i])
            self.pool_tags[p] = np.uint32((int(self.pool_tags[p]) + 1) & M32)
            if b not in stale:
                self.expected_tags[b, j] = self.pool_tags[p]
            bumped.append(p)
        return np.array(bumped, dtype=np.int64)

    @property
    def pages_allocated(self) -> np.ndarray:
        return self.notes["pages_allocated"]


def scales_from_amax(amax) -> np.ndarray:
    """fp32 scale = fp32(amax / 448), and 1.0 where amax is zero."""
    amax = np.asarray(amax, dtype=np.float32)
    s = amax / np.float32(448.0)
    return np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)


def _build(name, cfg_index, *, batch, layers, hq, hkv, d, page, seq_lens0, max_steps,
           pool_pages, k_sigma, v_sigma, q_sigma, garbage_tail, rng,
           partition_tokens=0, shuffle=True):
    """Allocate pages from a shuffled (or, if shuffle=False, in-order) pool and
    record matching tags."""
    seq_lens0 = np.asarray(seq_lens0, dtype=np.int32)
    need = [-(-(int(L) + max_steps) // page) for L in seq_lens0]
    total = sum(need)
    num_pages = pool_pages(total)
    assert num_pages >= total
    perm = rng.permutation(num_pages).astype(np.int32)
    if not shuffle:
        perm = np.arange(num_pages, dtype=np.int32)
    max_pages = max(need)
    if garbage_tail:
        bt = rng.integers(-(2 ** 31), 2 ** 31 - 1, size=(batch, max_pages), dtype=np.int64)
        bt = bt.astype(np.int32)
    else:
        bt = np.full((batch, max_pages), -1, dtype=np.int32)
    pool_tags = rng.integers(0, 2 ** 32, size=num_pages, dtype=np.uint64).astype(np.uint32)
    exp_tags = rng.integers(0, 2 ** 32, size=(batch, max_pages), dtype=np.uint64).astype(np.uint32)
    off = 0
    for b in range(batch):
        bt[b, :need[b]] = perm[off:off + need[b]]
        exp_tags[b, :need[b]] = pool_tags[bt[b, :need[b]]]
        off += need[b]
    wl = Workload(name=name, seed=1000 + cfg_index, batch=batch, num_layers=layers,
                  num_q_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=page,
                  seq_lens0=seq_lens0, block_table=bt, pool_tags=pool_tags,
                  expected_tags=exp_tags, num_pages=num_pages, k_sigma=k_sigma,
                  v_sigma=v_sigma, q_sigma=q_sigma, max_steps=max_steps,
                  partition_tokens=partition_tokens)
    wl.notes["pages_allocated"] = np.array(need, dtype=np.int64)
    return wl


def _rng(cfg_index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 + cfg_index))


def tiny_1req(max_steps: int = 1) -> Workload:
    """1 sequence, ctx 256 (appended token included), 16 pages of a 64-page pool.

    8 query heads / 1 KV head, head_dim 128, page 16, one layer; q, K, V all
    N(0, 1); random uint32 tags, all matching.
    """
    rng = _rng(0)
    return _build("tiny_1req", 0, batch=1, layers=1, hq=8, hkv=1, d=128, page=16,
                  seq_lens0=[255], max_steps=max_steps,
                  pool_pages=lambda total: max(64, total), k_sigma=1.0, v_sigma=1.0,
                  q_sigma=1.0, garbage_tail=False, rng=rng)


def mixed_8req(max_steps: int = 1) -> Workload:
    """8 sequences, ctx uniform in [1024, 8192], GQA 64/8, pool 2x, one stale tag."""
    rng = _rng(1)
    L = rng.integers(1024, 8192, size=8, endpoint=True)
    wl = _build("mixed_8req", 1, batch=8, layers=1, hq=64, hkv=8, d=128, page=16,
                seq_lens0=L - 1, max_steps=max_steps,
                pool_pages=lambda total: 2 * total, k_sigma=1.0, v_sigma=0.5,
                q_sigma=1.0, garbage_tail=True, rng=rng)
    sb = int(rng.integers(0, 8))
    j = int(rng.integers(0, wl.pages_of(sb, 0)))
    p = int(wl.block_table[sb, j])
    wl.pool_tags[p] = np.uint32((int(wl.pool_tags[p]) + 1) & M32)   # page reallocated
    wl.stale = (sb,)
    wl.notes["stale_page"] = (sb, j, p)
    return wl


def uniform_32req(max_steps: int = 1) -> Workload:
    """32 sequences, every ctx 8192, GQA 64/8, 8 layers; FP8 and BF16 caches."""
    rng = _rng(2)
    return _build("uniform_32req", 2, batch=32, layers=8, hq=64, hkv=8, d=128, page=16,
                  seq_lens0=np.full(32, 8191), max_steps=max_steps,
                  pool_pages=lambda total: total + 32, k_sigma=1.0, v_sigma=0.5,
                  q_sigma=1.0, garbage_tail=False, rng=rng)


def batch64_ctx8k(max_steps: int = 1) -> Workload:
    """64 sequences, ctx 8192 + uniform [0, 1000], GQA 64/8, 8 layers, FP8."""
    rng = _rng(3)
    L = 8192 + rng.integers(0, 1000, size=64, endpoint=True)
    return _build("batch64_ctx8k", 3, batch=64, layers=8, hq=64, hkv=8, d=128, page=16,
                  seq_lens0=L - 1, max_steps=max_steps,
                  pool_pages=lambda total: total + 64, k_sigma=1.0, v_sigma=0.5,
                  q_sigma=1.0, garbage_tail=False, rng=rng)


def concurrency_point(batch: int, max_steps: int = 1) -> Workload:
    """The first ``batch`` requests of the headline batch's length draw
    (8192 + uniform [0, 1000]), GQA 64/8, 8 layers: one point of the BF16 vs
    FP8 concurrency sweep."""
    rng = _rng(3)
    L = (8192 + rng.integers(0, 1000, size=64, endpoint=True))[:batch]
    return _build(f"concurrency_b{batch}", 5, batch=batch, layers=8, hq=64, hkv=8, d=128,
                  page=16, seq_lens0=L - 1, max_steps=max_steps,
                  pool_pages=lambda total: total + batch, k_sigma=1.0, v_sigma=0.5,
                  q_sigma=1.0, garbage_tail=False, rng=np.random.default_rng(1005 + batch))


def skewed_16req(max_steps: int = 2) -> Workload:
    """16 sequences, ctx log-uniform in [512, 131072] (two at 131072), 1 layer.

    Split-K partitions of 512 tokens; pool 1.25x; between steps 10% of the
    pages are freed and reallocated with a tag bump and two requests keep
    stale mappings (``stale`` lists them; they must abort after the churn).
    """
    rng = _rng(4)
    u = rng.uniform(np.log(512.0), np.log(131072.0), size=16)
    L = np.floor(np.exp(u)).astype(np.int64)
    L = np.clip(L, 512, 131072)
    L[0] = L[1] = 131072
    wl = _build("skewed_16req", 4, batch=16, layers=1, hq=64, hkv=8, d=128, page=16,
                seq_lens0=L - 1, max_steps=max_steps,
                pool_pages=lambda total: (5 * total + 3) // 4, k_sigma=1.0,
                v_sigma=0.5, q_sigma=1.0, garbage_tail=True, rng=rng,
                partition_tokens=512)
    wl.notes["churn_stale"] = tuple(int(x) for x in rng.choice(16, size=2, replace=False))
    wl.notes["churn_rng_seed"] = int(rng.integers(0, 2 ** 31))
    return wl


CONFIGS = {
    "tiny": tiny_1req,
    "mixed8": mixed_8req,
    "uniform32": uniform_32req,
    "batch64": batch64_ctx8k,
    "skewed16": skewed_16req,
}
