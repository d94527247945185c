"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments before enqueuing anything (no GPU needed: validation
precedes every HIP call). Also the header's tile layouts and the device twin
of the input hash."""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

import synth
from synth import device as sd
from tests.helpers import OFFSETS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]
LIB = os.path.join(ROOT, "fp8_e4m3_paged_amd", "libkvfp8.so")

OK, NULL, SHAPE, UNSUP, WORKSPACE, LAUNCH, ALIGN = 0, -1, -2, -3, -4, -5, -6


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


# Entry points that enqueue GPU work. The cases below pass fake device
# addresses, so every one of them must be refused by validation; a call that
# got through would launch a kernel on those addresses. On a host without a
# GPU such a call returns KV_ERR_LAUNCH, which the proxy turns into a failure.
LAUNCHING = {"kv_verify_tags", "kv_append_quant", "kv_append_bf16", "paged_decode_attn",
             "paged_decode_attn_append", "kv_amax_accumulate", "kv_scales_from_amax",
             "kv_ingest_prefill", "wq_quantize_pack", "wq_gemv"}


class _NoLaunch:
    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        fn = getattr(self._real, name)
        if name not in LAUNCHING:
            return fn

        def checked(*args):
            status = fn(*args)
            assert status != LAUNCH, f"{name}{args}: passed validation and reached a launch"
            return status
        return checked


@pytest.fixture(scope="module")
def real_lib():
    """The library itself, for calls that enqueue nothing."""
    if not os.path.exists(LIB):
        pytest.fail("libkvfp8.so not built: run python -m fp8_e4m3_paged_amd.build")
    import fp8_e4m3_paged_amd as k
    return k.load()


@pytest.fixture(scope="module")
def lib(real_lib):
    """The library behind the no-launch proxy, for the fake-address cases.
    Where a GPU is visible a call that wrongly passed validation would launch
    on those addresses, so these cases run only on hosts without one."""
    if torch.cuda.device_count() > 0:
        pytest.skip("fake device addresses are only passed where no GPU is visible")
    return _NoLaunch(real_lib)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["kv_verify_tags", "kv_append_quant", "kv_append_bf16", "paged_decode_attn",
              "paged_decode_attn_workspace_bytes", "paged_decode_attn_partition_tokens",
              "paged_decode_attn_append", "kv_amax_accumulate", "kv_scales_from_amax",
              "kv_ingest_prefill", "kv_status_str", "kv_pool_create", "kv_pool_destroy",
              "kv_pool_alloc", "kv_pool_free", "kv_pool_tags", "kv_pool_record_check",
              "kv_pool_get_stats", "wq_packed_bytes", "wq_quantize_pack", "wq_gemv",
              "paged_decode_attn_append_noalloc"]:
        assert n in names


def test_library_exports_every_declared_symbol(real_lib):
    raw = ctypes.CDLL(LIB)
    for n in declared_functions():
        assert hasattr(raw, n), n


def test_status_strings(real_lib):
    import fp8_e4m3_paged_amd as k
    for s in (OK, NULL, SHAPE, UNSUP, WORKSPACE, LAUNCH, ALIGN, -7, -8):
        assert k.kv_status_str(s).startswith("KV_")
    assert "unknown" in k.kv_status_str(42)


A = 1 << 20        # a fake, 16-byte aligned "device" address (never dereferenced)


def verify(lib, **kw):
    args = dict(pool_tags=A, num_pages=10, block_table=A, expected_tags=A, bt_stride=4,
                seq_lens=A, batch=2, page_size=16, abort_out=A, workspace=None,
                workspace_bytes=0, stream=None)
    args.update(kw)
    return lib.kv_verify_tags(*args.values())


def test_verify_rejects_bad_arguments(lib):
    assert verify(lib, page_size=8) == UNSUP
    assert verify(lib, batch=-1) == SHAPE
    assert verify(lib, bt_stride=-1) == SHAPE
    assert verify(lib, block_table=None) == NULL
    assert verify(lib, abort_out=None) == NULL
    assert verify(lib, seq_lens=A + 2) == ALIGN
    assert verify(lib, batch=0, block_table=None) == OK       # nothing to do
    # the split check's counters: one 64-bit word per request, only for rows
    # longer than one 2,048-page chunk
    assert lib.kv_verify_tags_workspace_bytes(3, 2048) == 0
    assert lib.kv_verify_tags_workspace_bytes(3, 2049) == 24
    assert lib.kv_verify_tags_workspace_bytes(0, 9000) == 0
    assert verify(lib, bt_stride=5000, workspace=A, workspace_bytes=8) == WORKSPACE
    assert verify(lib, bt_stride=5000, workspace=A + 4, workspace_bytes=16) == ALIGN
    assert verify(lib, batch=4_000_000, bt_stride=2_000_000, workspace=A,
                  workspace_bytes=1 << 40) == SHAPE       # 3.9e9 workgroups


def append(lib, fp8=True, **kw):
    args = dict(k_new=A, v_new=A, tok_seq=A, tok_pos=A, n_tok=3, block_table=A, bt_stride=4,
                batch=2)
    if fp8:
        args.update(k_scale=A, v_scale=A)
    args.update(k_pool=A, v_pool=A, num_pages=10, num_kv_heads=8, head_dim=128, page_size=16,
                abort=None, stream=None)
    args.update(kw)
    fn = lib.kv_append_quant if fp8 else lib.kv_append_bf16
    return fn(*args.values())


@pytest.mark.parametrize("fp8", [True, False])
def test_append_rejects_bad_arguments(lib, fp8):
    assert append(lib, fp8, head_dim=64) == UNSUP
    assert append(lib, fp8, page_size=32) == UNSUP
    assert append(lib, fp8, n_tok=-1) == SHAPE
    assert append(lib, fp8, num_kv_heads=0) == SHAPE
    assert append(lib, fp8, k_pool=None) == NULL
    assert append(lib, fp8, tok_pos=None) == NULL
    assert append(lib, fp8, v_new=A + 8) == ALIGN
    assert append(lib, fp8, n_tok=0, k_new=None) == OK
    if fp8:
        assert append(lib, fp8, k_scale=None) == NULL


def attn(lib, **kw):
    args = dict(q=A, cache_dtype=0, k_pool=A, v_pool=A, k_scale=A, v_scale=A, block_table=A,
                bt_stride=600, seq_lens=A, max_seq_len=9000, abort=None, out=A, sm_scale=0.088,
                batch=64, num_q_heads=64, num_kv_heads=8, head_dim=128, page_size=16,
                num_pages=40000, partition_tokens=0, workspace=A, workspace_bytes=1 << 40,
                stream=None)
    args.update(kw)
    return lib.paged_decode_attn(*args.values())


def test_attention_rejects_bad_arguments(lib):
    assert attn(lib, head_dim=64) == UNSUP
    assert attn(lib, page_size=8) == UNSUP
    assert attn(lib, num_q_heads=60) == SHAPE                 # not a multiple of 8
    assert attn(lib, num_q_heads=8 * 17) == UNSUP             # group of 17 > 16
    assert attn(lib, cache_dtype=7) == UNSUP
    assert attn(lib, partition_tokens=100) == UNSUP           # not a multiple of 16
    assert attn(lib, partition_tokens=32768) == UNSUP         # above the maximum
    assert attn(lib, batch=-2) == SHAPE
    assert attn(lib, q=None) == NULL
    assert attn(lib, k_scale=None) == NULL                    # FP8 needs scales
    assert attn(lib, out=A + 4) == ALIGN
    assert attn(lib, workspace=None, partition_tokens=512) == WORKSPACE
    assert attn(lib, workspace_bytes=16, partition_tokens=512) == WORKSPACE
    assert attn(lib, sm_scale=-0.5) == UNSUP
    assert attn(lib, sm_scale=float("nan")) == UNSUP
    assert attn(lib, sm_scale=float("inf")) == UNSUP
    assert attn(lib, batch=0, q=None) == OK


def attn_append(lib, k_new=A, v_new=A, **kw):
    args = dict(q=A, k_new=k_new, v_new=v_new, cache_dtype=0, k_pool=A, v_pool=A, k_scale=A,
                v_scale=A, block_table=A, bt_stride=600, seq_lens=A, max_seq_len=9000,
                abort=None, out=A, sm_scale=0.088, batch=64, num_q_heads=64, num_kv_heads=8,
                head_dim=128, page_size=16, num_pages=40000, partition_tokens=0, workspace=A,
                workspace_bytes=1 << 40, stream=None)
    args.update(kw)
    return lib.paged_decode_attn_append(*args.values())


def test_fused_append_attention_rejects_bad_arguments(lib):
    assert attn_append(lib, k_new=None) == NULL
    assert attn_append(lib, v_new=None) == NULL
    assert attn_append(lib, k_new=A + 2) == ALIGN
    assert attn_append(lib, v_new=A + 8) == ALIGN
    assert attn_append(lib, head_dim=64) == UNSUP
    assert attn_append(lib, k_scale=None) == NULL
    assert attn_append(lib, cache_dtype=1, k_scale=None, v_scale=None, out=A + 4) == ALIGN
    assert attn_append(lib, sm_scale=-1.0) == UNSUP
    assert attn_append(lib, workspace=None, partition_tokens=512) == WORKSPACE
    assert attn_append(lib, batch=0, k_new=None, v_new=None, q=None) == OK


def ingest_call(lib, **kw):
    args = dict(k_rows=A, v_rows=A, n_rows=1000, row_start=A, seq_lens=A, batch=4,
                max_seq_len=300, block_table=A, bt_stride=32, cache_dtype=0, k_scale=A,
                v_scale=A, k_pool=A, v_pool=A, num_pages=100, num_kv_heads=8, head_dim=128,
                page_size=16, abort=None, stream=None)
    args.update(kw)
    return lib.kv_ingest_prefill(*args.values())


def test_ingest_entry_points_reject_bad_arguments(lib):
    assert lib.kv_amax_accumulate(A, 10, 8, 64, A, None) == UNSUP
    assert lib.kv_amax_accumulate(A, -1, 8, 128, A, None) == SHAPE
    assert lib.kv_amax_accumulate(A, 10, 0, 128, A, None) == SHAPE
    assert lib.kv_amax_accumulate(None, 10, 8, 128, A, None) == NULL
    assert lib.kv_amax_accumulate(A + 8, 10, 8, 128, A, None) == ALIGN
    assert lib.kv_amax_accumulate(None, 0, 8, 128, None, None) == OK      # nothing to do
    assert lib.kv_scales_from_amax(A, -1, A, None) == SHAPE
    assert lib.kv_scales_from_amax(None, 4, A, None) == NULL
    assert lib.kv_scales_from_amax(A, 4, A + 2, None) == ALIGN
    assert lib.kv_scales_from_amax(None, 0, None, None) == OK
    assert ingest_call(lib, head_dim=64) == UNSUP
    assert ingest_call(lib, page_size=32) == UNSUP
    assert ingest_call(lib, cache_dtype=3) == UNSUP
    assert ingest_call(lib, n_rows=-1) == SHAPE
    assert ingest_call(lib, num_pages=-1) == SHAPE
    assert ingest_call(lib, bt_stride=-3) == SHAPE
    assert ingest_call(lib, k_scale=None) == NULL                          # FP8 needs scales
    # BF16 takes no scales: NULL passes the pointer checks (stopped here by the alignment one)
    assert ingest_call(lib, cache_dtype=1, k_scale=None, v_scale=None, v_pool=A + 4) == ALIGN
    assert ingest_call(lib, row_start=None) == NULL
    assert ingest_call(lib, k_pool=A + 4) == ALIGN
    assert ingest_call(lib, batch=0, k_rows=None) == OK


def test_weight_gemv_entry_points_reject_bad_arguments(lib):
    assert lib.wq_packed_bytes(64, 256, 0) == 64 * 256 // 2
    assert lib.wq_packed_bytes(64, 256, 1) == 64 * 256
    assert lib.wq_packed_bytes(60, 256, 0) == 0 and lib.wq_packed_bytes(64, 200, 1) == 0
    assert lib.wq_packed_bytes(64, 256, 5) == 0
    assert lib.wq_quantize_pack(A, 60, 256, 0, A, A, None) == UNSUP      # rows % 16
    assert lib.wq_quantize_pack(A, 64, 100, 0, A, A, None) == UNSUP      # inputs % 128
    assert lib.wq_quantize_pack(A, 64, 256, 2, A, A, None) == UNSUP      # format
    assert lib.wq_quantize_pack(A, -16, 256, 0, A, A, None) == SHAPE
    assert lib.wq_quantize_pack(None, 64, 256, 0, A, A, None) == NULL
    assert lib.wq_quantize_pack(A, 64, 256, 0, A + 4, A, None) == ALIGN
    assert lib.wq_quantize_pack(None, 0, 256, 0, None, None, None) == OK
    assert lib.wq_gemv(A, 4, A, A, 64, 256, 0, None, None) == NULL
    assert lib.wq_gemv(A, 4, A, A, 64, 256, 0, A + 8, None) == ALIGN
    assert lib.wq_gemv(A, -1, A, A, 64, 256, 0, A, None) == SHAPE
    assert lib.wq_gemv(A, 4, A, A, 72, 256, 0, A, None) == UNSUP
    assert lib.wq_gemv(None, 0, None, None, 64, 256, 1, None, None) == OK


def test_workspace_and_partition_sizing(real_lib):
    import fp8_e4m3_paged_amd as k
    # one partition covers everything: no workspace
    assert k.paged_decode_attn_workspace_bytes(64, 64, 8, 8000, 8192) == 0
    # 16 requests, 64 heads, up to 131073 tokens at 512 -> 257 partitions, and
    # one more partial slot per (request, query head) for the wave-mode kernel:
    # the (max, sum) pairs, then the outputs from the next 256-byte boundary
    n = 16 * 64 * (257 + 1)
    ml = -(-(n * 2 * 4) // 256) * 256
    assert k.paged_decode_attn_workspace_bytes(16, 64, 8, 131073, 512) == ml + n * 128 * 4
    n = 3 * 4 * (3 + 1)
    assert k.paged_decode_attn_workspace_bytes(3, 4, 2, 3 * 1024, 1024) == \
        -(-(n * 2 * 4) // 256) * 256 + n * 128 * 4
    for cd in (k.KV_CACHE_FP8_E4M3, k.KV_CACHE_BF16):
        for b, h, L in [(64, 8, 9193), (1, 1, 256), (16, 8, 131073), (8, 8, 8192)]:
            pt = k.paged_decode_attn_partition_tokens(b, h, L, 0, cd)
            assert pt % 16 == 0 and 16 <= pt <= 16384
        assert k.paged_decode_attn_partition_tokens(64, 8, 9193, 512, cd) == 512
        with pytest.raises(k.KvError):
            k.paged_decode_attn_partition_tokens(64, 8, 9193, 24, cd)
    # automatic: at most 16 equal shares rounded up to 256 tokens (to a page
    # pair where that would drop partitions), each at least 192 KiB of K and V
    # per KV head (768 FP8 tokens, 384 BF16 tokens)
    assert k.paged_decode_attn_partition_tokens(1, 8, 9193, 0, k.KV_CACHE_FP8_E4M3) == 768
    assert k.paged_decode_attn_partition_tokens(1, 8, 9193, 0, k.KV_CACHE_BF16) == 576
    assert k.paged_decode_attn_partition_tokens(8, 8, 9193, 0, k.KV_CACHE_BF16) == 2304
    assert k.paged_decode_attn_partition_tokens(8, 8, 9082, 0, k.KV_CACHE_FP8_E4M3) == 2304
    assert k.paged_decode_attn_partition_tokens(4, 8, 8797, 0, k.KV_CACHE_FP8_E4M3) == 1120
    assert k.paged_decode_attn_partition_tokens(64, 8, 9193, 0, k.KV_CACHE_FP8_E4M3) == 9216
    # the BF16 size at one request: 16 partitions (+1 slot) per (request, query head)
    n = 1 * 64 * (16 + 1)
    assert k.paged_decode_attn_workspace_bytes(1, 64, 8, 9193, 0, cache_dtype=k.KV_CACHE_BF16) \
        == -(-(n * 2 * 4) // 256) * 256 + n * 128 * 4
    with pytest.raises(k.KvError):
        k.paged_decode_attn_partition_tokens(1, 8, 9193, 0, 7)
    assert k.paged_decode_attn_workspace_bytes(1, 64, 8, 9193, 0, cache_dtype=7) == 0


@pytest.mark.parametrize("key", sorted(OFFSETS))
def test_tile_layouts_are_permutations(key):
    off = OFFSETS[key]
    assert sorted(off.ravel().tolist()) == list(range(16 * 128))


def test_device_hash_twin_matches_host_on_cpu_torch():
    wl = synth.mixed_8req()
    seq = torch.tensor([0, 3, 3, 7], dtype=torch.int32)
    pos = torch.tensor([0, 5, 1500, int(wl.seq_lens0[7])], dtype=torch.int32)
    for kind in ("k", "v"):
        got = sd.kv_bits_tokens(wl, 0, kind, seq, pos).numpy().view(np.uint16)
        for i in range(4):
            b, t = int(seq[i]), int(pos[i])
            assert np.array_equal(got[i], wl.kv_bits(0, kind, b, t, t + 1)[0])


def test_launch_size_limits_are_refused_before_anything_is_enqueued(lib):
    """One launch holds at most 2^32 - 1 work-items: sizes that would need more
    return KV_ERR_SHAPE. Each limit is probed just above (refused) and just
    below, where the call must get past the size check and stop at a later
    one (a NULL pointer or a small workspace), so nothing is ever launched."""
    # tag check: one 1024-thread workgroup per request
    assert verify(lib, batch=4_194_304) == SHAPE
    assert verify(lib, batch=4_194_303, block_table=None) == NULL
    # append: one row of 256-thread workgroups per token
    assert append(lib, n_tok=16_777_216) == SHAPE
    assert append(lib, n_tok=16_777_215, k_pool=None) == NULL
    # attention: one workgroup (<= 512 threads) per (partition, request, KV head)
    assert attn(lib, batch=1_048_577) == SHAPE                 # one partition, 8 KV heads
    assert attn(lib, batch=1_048_575, q=None) == NULL
    # ... and the reduce, held to 512 work-items per (request, query head)
    assert attn(lib, batch=600_000, num_q_heads=16, num_kv_heads=1, max_seq_len=1024,
                partition_tokens=512) == SHAPE
    assert attn(lib, batch=500_000, num_q_heads=16, num_kv_heads=1, max_seq_len=1024,
                partition_tokens=512, workspace_bytes=16) == WORKSPACE
    # weight packing: one wavefront per (16-row tile, 128-input group)
    assert lib.wq_quantize_pack(A, 16_777_216, 8192, 0, A, A, None) == SHAPE
    assert lib.wq_quantize_pack(None, 16_777_216, 8064, 0, A, A, None) == NULL
    # GEMV: at most one workgroup per (64-row group, 128-input group)
    assert lib.wq_gemv(A, 1, A, A, 16_777_216, 8192, 0, A, None) == SHAPE
    assert lib.wq_gemv(None, 1, A, A, 16_777_216, 8064, 0, A, None) == NULL
