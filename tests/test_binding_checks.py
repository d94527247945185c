"""The Python binding checks tensor sizes against each other before it takes
any pointer: the C ABI sees only raw pointers, and the kernels index the
request arrays by batch, the scales by KV head and the pools by whole
(page, KV head) tiles, so a short or misshaped tensor would be read past its
end on the GPU. On the host every such call must stop with a ValueError that
names the tensor; a call whose sizes agree gets as far as the device check."""

import pytest
import torch

import fp8_e4m3_paged_amd as kv

B, HQ, HKV, D, P = 4, 16, 2, 128, 16


def _attn_args(**over):
    a = dict(q=torch.zeros(B, HQ, D, dtype=torch.bfloat16),
             k_pool=torch.zeros(10, HKV, P, D, dtype=torch.uint8),
             v_pool=torch.zeros(10, HKV, P, D, dtype=torch.uint8),
             k_scale=torch.ones(HKV), v_scale=torch.ones(HKV),
             block_table=torch.zeros(B, 3, dtype=torch.int32),
             seq_lens=torch.ones(B, dtype=torch.int32), max_seq_len=48,
             out=torch.zeros(B, HQ, D), sm_scale=0.088)
    a.update(over)
    return a


def _call_attn(**over):
    a = _attn_args(**over)
    kv.paged_decode_attn(a["q"], a["k_pool"], a["v_pool"], a["k_scale"], a["v_scale"],
                         a["block_table"], a["seq_lens"], a["max_seq_len"], a["out"],
                         a["sm_scale"], abort=a.get("abort"))


@pytest.mark.parametrize("over,msg", [
    (dict(seq_lens=torch.ones(B - 1, dtype=torch.int32)), "seq_lens"),
    (dict(block_table=torch.zeros(B + 1, 3, dtype=torch.int32)), "block_table"),
    (dict(abort=torch.zeros(B - 2, dtype=torch.uint8)), "abort"),
    (dict(k_scale=torch.ones(HKV + 1)), "k_scale"),
    (dict(v_pool=torch.zeros(11, HKV, P, D, dtype=torch.uint8)), "alike"),
    (dict(k_pool=torch.zeros(10, HKV, P, 64, dtype=torch.uint8),
          v_pool=torch.zeros(10, HKV, P, 64, dtype=torch.uint8)), "bytes per"),
])
def test_attention_sizes_are_checked(over, msg):
    kv.load()
    with pytest.raises(ValueError, match=msg):
        _call_attn(**over)


def test_consistent_sizes_reach_the_device_check():
    kv.load()
    with pytest.raises(ValueError, match="GPU tensor"):
        _call_attn()


def test_fused_append_and_append_sizes_are_checked():
    kv.load()
    a = _attn_args()
    k_new = torch.zeros(B, HKV, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="seq_lens"):
        kv.paged_decode_attn_append(a["q"], k_new, k_new, a["k_pool"], a["v_pool"],
                                    a["k_scale"], a["v_scale"], a["block_table"],
                                    torch.ones(B + 3, dtype=torch.int32), 48, a["out"], 0.088)
    with pytest.raises(ValueError, match="bytes per"):
        kv.kv_append_bf16(k_new, k_new, torch.zeros(B, dtype=torch.int32),
                          torch.zeros(B, dtype=torch.int32), a["block_table"],
                          a["k_pool"], a["v_pool"])            # FP8-sized tiles for BF16
    with pytest.raises(ValueError, match="abort"):
        kv.kv_append_quant(k_new, k_new, torch.zeros(B, dtype=torch.int32),
                           torch.zeros(B, dtype=torch.int32), a["block_table"], a["k_scale"],
                           a["v_scale"], a["k_pool"], a["v_pool"],
                           abort=torch.zeros(B + 1, dtype=torch.uint8))


def test_ingest_and_gemv_sizes_are_checked():
    kv.load()
    rows = torch.zeros(40, HKV, D, dtype=torch.bfloat16)
    a = _attn_args()
    with pytest.raises(ValueError, match="v_scale"):
        kv.kv_ingest_prefill(rows, rows, torch.zeros(B, dtype=torch.int32), a["seq_lens"],
                             a["block_table"], a["k_pool"], a["v_pool"], 48, a["k_scale"],
                             torch.ones(HKV + 2))
    with pytest.raises(ValueError, match="row_start"):
        kv.kv_ingest_prefill(rows, rows, torch.zeros(B + 1, dtype=torch.int32), a["seq_lens"],
                             a["block_table"], a["k_pool"], a["v_pool"], 48, a["k_scale"],
                             a["v_scale"])
    x = torch.zeros(1, 256, dtype=torch.bfloat16)
    y = torch.zeros(1, 64)
    packed = torch.zeros(kv.wq_packed_bytes(64, 256, kv.WQ_INT4) - 16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="packed"):
        kv.wq_gemv(x, packed, torch.zeros(64 * 2), y, 64, kv.WQ_INT4)
    packed = torch.zeros(kv.wq_packed_bytes(64, 256, kv.WQ_INT4), dtype=torch.uint8)
    with pytest.raises(ValueError, match="scales"):
        kv.wq_gemv(x, packed, torch.zeros(64), y, 64, kv.WQ_INT4)


def test_prepare_checks_sizes_like_a_direct_call():
    """prepare=True runs the same checks before it builds anything."""
    a = _attn_args(seq_lens=torch.ones(B - 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="seq_lens"):
        kv.paged_decode_attn(a["q"], a["k_pool"], a["v_pool"], a["k_scale"], a["v_scale"],
                             a["block_table"], a["seq_lens"], a["max_seq_len"], a["out"],
                             a["sm_scale"], prepare=True)


def test_prepared_call_raises_what_the_library_refuses():
    """A Prepared whose fixed arguments the C ABI refuses raises KvError with
    that status on every call (a negative batch is refused before any HIP
    call, so this runs without a GPU)."""
    lib = kv.load()
    args = (None, None, None, 0, None, None, None, None, None, 3, None, 48, None, None, 0.088,
            -1, HQ, HKV, D, P, 10, 0, None, 0, None)
    call = kv.Prepared("paged_decode_attn_append", lib.paged_decode_attn_append, args, ())
    for _ in range(2):
        with pytest.raises(kv.KvError) as e:
            call()
        assert e.value.status == -2            # KV_ERR_SHAPE
