"""GPU parity of the weight-only quantized decode GEMV (wq_quantize_pack,
wq_gemv) against the oracle in oracle/weights.py: codes and scales bit for
bit (unpacked through the layout formulas of include/kvfp8.h, written out
here independently), the product within a tolerance derived from fp32
accumulation of exact products."""

import numpy as np
import pytest
import torch

from oracle import weights
from tests.gpu_harness import DEV, say

pytestmark = pytest.mark.gpu
G = 128
# fp32 sums of exact bf16 x int products, 128 per group, then scaled groups:
# relative error well below 1e-5 of the result's norm
REL_TOL = 1e-5


@pytest.fixture(scope="module")
def kv():
    import fp8_e4m3_paged_amd as k
    k.load()
    return k


def _index_maps(n, k, fmt):
    """Byte offset of every element (row, input), from the header's formulas; INT4:
    the offset of its dword and the value index i within it."""
    rows = np.arange(n)[:, None]
    cols = np.arange(k)[None, :]
    nt, r = rows // 16, rows % 16
    g, kk = cols // G, cols % G
    c, j, i = kk // 32, (kk % 32) // 8, kk % 8
    b = nt * (k // G) + g
    lane = 16 * j + r
    if fmt == 0:
        return 1024 * b + 16 * lane + 4 * c, i
    return 2048 * b + 1024 * (c // 2) + 16 * lane + 8 * (c % 2) + i, None


def _unpack(packed, n, k, fmt):
    off, i = _index_maps(n, k, fmt)
    if fmt == 0:
        # the header's fields: i < 4: |q| in bits 0..2, sign in bit 7 of byte i;
        # i >= 4: |q| in bits 4..6 of byte i % 4, sign in bit 3 of byte (i + 1) % 4
        word = packed.view(np.uint32)[off // 4].astype(np.int64)
        j = i % 4
        mag = np.where(i < 4, word >> (8 * j), word >> (8 * j + 4)) & 7
        neg = np.where(i < 4, word >> (8 * j + 7), word >> (8 * ((j + 1) % 4) + 3)) & 1
        assert not np.any((neg == 1) & (mag == 0)), "negative zero code"
        return np.where(neg == 1, -mag, mag).astype(np.int8)
    return packed[off]


def _weights(rng, n, k):
    w = rng.normal(0, 0.03, size=(n, k)).astype(np.float32)
    bits = (w.view(np.uint32) >> 16).astype(np.uint16)
    # an all-zero group, and a group of exact multiples with ties (2.5 s, 3.5 s, ...)
    bits[0, :G] = 0
    if n > 1 and k >= 2 * G:
        ties = np.array([7.0, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5] * (G // 8)) * 2.0 ** -6
        bits[1, G:2 * G] = (ties.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return bits


def _pack(kv, wb, fmt):
    n, k = wb.shape
    w = torch.from_numpy(wb.view(np.int16)).to(DEV)
    packed = torch.zeros(kv.wq_packed_bytes(n, k, fmt), dtype=torch.uint8, device=DEV)
    scales = torch.zeros(n * (k // G), dtype=torch.float32, device=DEV)
    kv.wq_quantize_pack(w, packed, scales, fmt)
    torch.cuda.synchronize()
    return packed, scales


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("n,k", [(16, 128), (64, 256), (80, 384), (1024, 1024)])
def test_pack_codes_and_scales_bit_exact(kv, fmt, n, k):
    wb = _weights(np.random.default_rng(n + k + fmt), n, k)
    packed, scales = _pack(kv, wb, fmt)
    q_o, s_o = weights.quantize_int4(wb) if fmt == 0 else weights.quantize_fp8(wb)
    got_s = scales.cpu().numpy().reshape(n // 16, k // G, 16).transpose(0, 2, 1).reshape(n, k // G)
    assert np.array_equal(got_s.view(np.uint32), s_o.view(np.uint32))
    got_q = _unpack(packed.cpu().numpy(), n, k, fmt)
    assert np.array_equal(got_q, q_o)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("m", [1, 2, 5, 8, 9, 16, 17, 33, 64, 70])
@pytest.mark.parametrize("n,k", [(320, 1024), (336, 1152)])
def test_gemv_against_oracle(kv, fmt, m, n, k):
    """1 .. 4 tokens take the small-batch kernel, more the chunked one; 336 x
    1152 has a last group of 64 rows with one tile and input ranges of
    unequal length."""
    rng = np.random.default_rng(100 + m + fmt + n)
    wb = _weights(rng, n, k)
    packed, scales = _pack(kv, wb, fmt)
    q_o, s_o = weights.quantize_int4(wb) if fmt == 0 else weights.quantize_fp8(wb)
    wd = weights.dequant_int4(q_o, s_o) if fmt == 0 else weights.dequant_fp8(q_o, s_o)
    xb = (rng.normal(0, 1, size=(m, k)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bias = rng.normal(0, 1, size=(m, n)).astype(np.float32)
    y = torch.from_numpy(bias.copy()).to(DEV)
    kv.wq_gemv(torch.from_numpy(xb.view(np.int16)).to(DEV), packed, scales, y, n, fmt)
    torch.cuda.synchronize()
    want = bias.astype(np.float64) + weights.gemv(xb, wd)
    got = y.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert rel <= REL_TOL, f"fmt {fmt} m {m}: rel_l2 {rel:.2e}"


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("m", [1, 4, 64])
def test_one_hot_inputs_read_every_code_position(kv, fmt, m):
    """Token t of a call has x = 1.0 at one input j_t and zeros elsewhere, and
    the calls run j over every input of a 32 x 256 matrix, so each output is a
    single product: y[t] must equal fp32(q[:, j_t] * s) bit for bit. INT4
    weights are q * 2^-6 with q = (3 row + input) % 15 - 7, so every code value
    sits at every position of the packed words and each group's scale is
    exactly 2^-6; FP8 weights are random. 1 and 4 tokens take the small-batch
    kernel, 64 the chunked one."""
    n, k = 32, 2 * G
    if fmt == 0:
        q = ((3 * np.arange(n)[:, None] + np.arange(k)[None, :]) % 15 - 7).astype(np.float32)
        wb = ((q * 2.0 ** -6).view(np.uint32) >> 16).astype(np.uint16)
    else:
        wb = _weights(np.random.default_rng(11), n, k)
    packed, scales = _pack(kv, wb, fmt)
    q_o, s_o = weights.quantize_int4(wb) if fmt == 0 else weights.quantize_fp8(wb)
    if fmt == 0:
        assert np.array_equal(q_o, q.astype(q_o.dtype)) and np.all(s_o == 2.0 ** -6)
    assert np.array_equal(_unpack(packed.cpu().numpy(), n, k, fmt), q_o)
    wd = weights.dequant_int4(q_o, s_o) if fmt == 0 else weights.dequant_fp8(q_o, s_o)
    want_cols = wd.astype(np.float32)            # one exact product, rounded once to fp32
    for j0 in range(0, k, m):
        cols = (j0 + np.arange(m)) % k
        xb = np.zeros((m, k), np.uint16)
        xb[np.arange(m), cols] = 0x3F80                                 # bf16 1.0
        y = torch.zeros((m, n), dtype=torch.float32, device=DEV)
        kv.wq_gemv(torch.from_numpy(xb.view(np.int16)).to(DEV), packed, scales, y, n, fmt)
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        want = want_cols[:, cols].T
        assert np.array_equal(got, want), f"fmt {fmt} m {m} inputs {cols[:4]}..: " \
            f"{np.argwhere(got != want)[:4].tolist()}"


def _full_size_check(kv, fmt, m, n, k, seed):
    """Every code, scale and output of an n x k product at m tokens, in the
    launch configuration the benchmark times, against the oracle."""
    rng = np.random.default_rng(seed)
    wb = _weights(rng, n, k)
    packed, scales = _pack(kv, wb, fmt)
    xb = (rng.normal(0, 1, size=(m, k)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = torch.zeros((m, n), dtype=torch.float32, device=DEV)
    kv.wq_gemv(torch.from_numpy(xb.view(np.int16)).to(DEV), packed, scales, y, n, fmt)
    torch.cuda.synchronize()
    q_o, s_o = weights.quantize_int4(wb) if fmt == 0 else weights.quantize_fp8(wb)
    assert np.array_equal(_unpack(packed.cpu().numpy(), n, k, fmt), q_o), "codes"
    got_s = scales.cpu().numpy().reshape(n // 16, k // G, 16).transpose(0, 2, 1).reshape(n, k // G)
    assert np.array_equal(got_s.view(np.uint32), s_o.view(np.uint32)), "scales"
    del wb, packed, scales
    wd = weights.dequant_int4(q_o, s_o) if fmt == 0 else weights.dequant_fp8(q_o, s_o)
    want = weights.gemv(xb, wd)
    got = y.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(got - want, axis=1) / np.linalg.norm(want, axis=1)
    assert np.all(rel <= REL_TOL), rel
    say(f"gemv fmt {fmt} {n}x{k} m={m}: every code, scale and output; worst token rel_l2 "
        f"{rel.max():.2e}")


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("m", [1, 16])
def test_gemv_full_size_every_output(kv, fmt, m):
    """8192 x 8192 weights, 1 token (the small-batch kernel) and 16 tokens
    (the chunked kernel): every code and scale bit for bit, every output
    within the tolerance (per token)."""
    _full_size_check(kv, fmt, m, 8192, 8192, 7 + fmt)


def test_gemv_largest_product_every_output(kv):
    """The 28672 x 8192 INT4 product at one token, the roofline launch: every
    code, scale and output against the oracle."""
    _full_size_check(kv, 0, 1, 28672, 8192, 11)
