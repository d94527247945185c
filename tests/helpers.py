"""Test-side helpers: the pool tile layout as the C header documents it, oracle
pools built on the host, and the parity tolerance check.

The layout formulas are written here from the header's text, independently of
the library's own implementation, so that the bit-exact pool comparison also
checks that the library stores each element where it says it does.
"""

from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import e4m3  # noqa: E402

P, D = 16, 128

REL_L2_TOL = 1e-3
MAX_ABS_TOL = 5e-3


def _offsets(kind: str, cache: str) -> np.ndarray:
    """offsets[t, d] = element index inside one tile (bytes for FP8, bf16 words for BF16)."""
    t = np.arange(P)[:, None]
    d = np.arange(D)[None, :]
    if cache == "fp8":
        if kind == "k":
            off = 1024 * ((d % 32) // 16) + 256 * (d // 32) + 16 * t + (d % 16)
        else:
            off = 1024 * (d // 64) + 256 * (t // 4) + 16 * (d % 16) + 4 * ((d // 16) % 4) + (t % 4)
        return off
    if kind == "k":
        off = 1024 * ((d % 32) // 8) + 256 * (d // 32) + 16 * t + 2 * (d % 8)
    else:
        off = 1024 * (d // 32) + 256 * (t // 4) + 16 * (d % 16) + 8 * ((d // 16) % 2) + 2 * (t % 4)
    return off // 2


OFFSETS = {(k, c): _offsets(k, c) for k in ("k", "v") for c in ("fp8", "bf16")}


def tiles_to_logical(tiles: np.ndarray, kind: str, cache: str) -> np.ndarray:
    """[..., 2048] device tiles -> [..., 16, 128] logical (token, dim) arrays."""
    off = OFFSETS[(kind, cache)]
    return tiles[..., off]


def logical_to_tiles(logical: np.ndarray, kind: str, cache: str) -> np.ndarray:
    off = OFFSETS[(kind, cache)]
    out = np.zeros(logical.shape[:-2] + (P * D,), dtype=logical.dtype)
    out[..., off] = logical
    return out


def oracle_pools(wl, layer: int, k_scale, v_scale, cache: str = "fp8"):
    """Logical pools [num_pages][Hkv][16][128] holding every initial token,
    quantized by the oracle (FP8) or copied (BF16); unwritten slots are 0."""
    dt = np.uint8 if cache == "fp8" else np.uint16
    shape = (wl.num_pages, wl.num_kv_heads, P, D)
    kp, vp = np.zeros(shape, dt), np.zeros(shape, dt)
    for b in range(wl.batch):
        L = int(wl.seq_lens0[b])
        if L == 0:
            continue
        kb = wl.kv_bits(layer, "k", b, 0, L)
        vb = wl.kv_bits(layer, "v", b, 0, L)
        if cache == "fp8":
            kb = e4m3.quantize(kb, np.asarray(k_scale)[None, :, None])
            vb = e4m3.quantize(vb, np.asarray(v_scale)[None, :, None])
        for j in range(-(-L // P)):
            page = int(wl.block_table[b, j])
            n = min(P, L - j * P)
            kp[page, :, :n, :] = kb[j * P:j * P + n].transpose(1, 0, 2)
            vp[page, :, :n, :] = vb[j * P:j * P + n].transpose(1, 0, 2)
    return kp, vp


def request_codes(wl, layer, b, L, k_scale, v_scale, cache="fp8"):
    """Oracle's logical [Hkv][L][D] codes (or bf16 bits) of one request's first L tokens."""
    kb = wl.kv_bits(layer, "k", b, 0, L)
    vb = wl.kv_bits(layer, "v", b, 0, L)
    if cache == "fp8":
        kb = e4m3.quantize(kb, np.asarray(k_scale)[None, :, None])
        vb = e4m3.quantize(vb, np.asarray(v_scale)[None, :, None])
    return kb.transpose(1, 0, 2), vb.transpose(1, 0, 2)


def gather_device_request(pool_host_tiles, block_table_row, L, kind, cache):
    """Logical [Hkv][L][D] of one request read from device tiles copied to the host."""
    n = -(-L // P)
    tiles = pool_host_tiles[np.asarray(block_table_row[:n], dtype=np.int64)]   # [n][Hkv][2048]
    lg = tiles_to_logical(tiles, kind, cache)                                  # [n][Hkv][16][128]
    hkv = lg.shape[1]
    return lg.transpose(1, 0, 2, 3).reshape(hkv, n * P, D)[:, :L]


def attention_errors(got: np.ndarray, want: np.ndarray):
    """Per-row errors of [..., D] outputs: (rel-L2 of each row, max |err| of
    each row, rel-L2 over everything). A row whose reference is all zeros has
    rel-L2 0 if it is matched exactly, else infinity."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = got - want
    en = np.linalg.norm(err, axis=-1)
    wn = np.linalg.norm(want, axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(wn > 0, en / np.where(wn > 0, wn, 1.0), np.where(en > 0, np.inf, 0.0))
    mx = np.abs(err).max(axis=-1) if err.size else np.zeros(err.shape[:-1])
    glob = np.linalg.norm(err) / max(np.linalg.norm(want), 1e-300)
    return rel, mx, glob


def check_attention(got: np.ndarray, want: np.ndarray, zero_rows=(), label=""):
    """The attention tolerance, applied to every (request, query head) row on
    its own: rel-L2 <= 1e-3 and max |err| <= 5e-3 for each row of the
    non-aborted requests, so an error confined to one request or one head
    (a dropped or misplaced token) is not diluted by the exact rows around
    it. Requests listed in zero_rows must be exactly 0. ``got`` / ``want``
    are [requests][heads][D]. Returns (worst row rel-L2, worst max |err|);
    the rel-L2 over all rows is reported in the failure message only."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    keep = np.ones(got.shape[0], dtype=bool)
    for b in zero_rows:
        assert np.all(got[b] == 0.0), f"{label}: request {b} must be all zeros"
        keep[b] = False
    g, w = got[keep], want[keep]
    assert np.all(np.isfinite(g)), f"{label}: non-finite output"
    if g.size == 0:
        return 0.0, 0.0
    rel, mx, glob = attention_errors(g, w)
    worst = np.unravel_index(int(np.argmax(rel)), rel.shape)
    rows = np.flatnonzero(keep)
    where = f"request {rows[worst[0]]}" + (f" head {worst[1]}" if len(worst) > 1 else "")
    ok = (rel <= REL_L2_TOL) & (mx <= MAX_ABS_TOL)
    assert np.all(ok), (f"{label}: {int((~ok).sum())} rows out of tolerance; worst {where}: "
                        f"rel_l2={rel.max():.3e}, max_abs={mx.max():.3e} "
                        f"(all rows together: rel_l2={glob:.3e})")
    return float(rel.max()), float(mx.max())
