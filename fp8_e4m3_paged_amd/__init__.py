"""Python binding of libkvfp8.so: paged FP8-e4m3 KV-cache decode on MI355X.

A thin ctypes layer over the C ABI declared in include/kvfp8.h. Each function
takes torch tensors that already live on the GPU, checks their dtypes and
shapes, and passes raw device pointers plus the current HIP stream of torch.
Every step of the computation runs in the library's HIP kernels; there is no
fallback: if the shared library is not built, importing this package still
works but the first call raises ``KvLibraryMissing``.

Entry points (same names as the C ABI):
    kv_verify_tags, kv_verify_tags_workspace_bytes, kv_append_quant, kv_append_bf16,
    paged_decode_attn,
    paged_decode_attn_append, paged_decode_attn_append_noalloc,
    paged_decode_attn_workspace_bytes, paged_decode_attn_partition_tokens, kv_amax_accumulate,
    kv_scales_from_amax, kv_ingest_prefill, kv_status_str
and the weight-only quantized decode GEMV: wq_packed_bytes, wq_quantize_pack,
wq_gemv;
plus ``decode_step``, which enqueues one decode step (tag check, then per
layer append and attention) in the order the operations require, and
``ingest_layer``, which calibrates one layer's scales and writes its prompts.
The decode entry points also take ``prepare=True``, which checks the call
once and returns it as a ``Prepared`` to be enqueued again at the cost of the
C call alone.
``PagePool`` wraps the host page pool and tag tracker of include/kvpool.h
(kv_pool_create, kv_pool_alloc, kv_pool_free, kv_pool_tags,
kv_pool_record_check, kv_pool_get_stats, kv_pool_destroy).
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "KV_CACHE_FP8_E4M3", "KV_CACHE_BF16", "KvError", "KvLibraryMissing", "lib_path",
    "load", "kv_status_str", "kv_verify_tags", "kv_verify_tags_workspace_bytes",
    "kv_append_quant", "kv_append_bf16",
    "paged_decode_attn", "paged_decode_attn_append", "paged_decode_attn_workspace_bytes",
    "paged_decode_attn_append_noalloc", "KV_NOALLOC_SCRATCH_BYTES",
    "paged_decode_attn_partition_tokens", "decode_step", "PAGE_SIZE", "HEAD_DIM",
    "kv_amax_accumulate", "kv_scales_from_amax", "kv_ingest_prefill", "ingest_layer",
    "PagePool", "KV_ERR_EXHAUSTED", "KV_ERR_STATE",
    "WQ_INT4", "WQ_FP8_E4M3", "wq_packed_bytes", "wq_quantize_pack", "wq_gemv", "Prepared",
]

WQ_INT4 = 0
WQ_FP8_E4M3 = 1

KV_ERR_EXHAUSTED = -7
KV_ERR_STATE = -8

KV_CACHE_FP8_E4M3 = 0
KV_CACHE_BF16 = 1
PAGE_SIZE = 16
HEAD_DIM = 128
KV_NOALLOC_SCRATCH_BYTES = 64 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class KvError(RuntimeError):
    """A C-ABI call returned a negative kv_status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {kv_status_str(status)} ({status})")


class KvLibraryMissing(RuntimeError):
    """libkvfp8.so has not been built (python -m fp8_e4m3_paged_amd.build)."""


def lib_path() -> str:
    return os.environ.get("KVFP8_LIB", os.path.join(_HERE, "libkvfp8.so"))


_P = ctypes.c_void_p
_I = ctypes.c_int32
_L = ctypes.c_int64
_SIGS = {
    "kv_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "kv_verify_tags": (ctypes.c_int, [_P, _I, _P, _P, _I, _P, _I, _I, _P, _P, ctypes.c_size_t,
                                      _P]),
    "kv_verify_tags_workspace_bytes": (ctypes.c_size_t, [_I, _I]),
    "kv_append_quant": (ctypes.c_int, [_P, _P, _P, _P, _I, _P, _I, _I, _P, _P, _P, _P, _I,
                                       _I, _I, _I, _P, _P]),
    "kv_append_bf16": (ctypes.c_int, [_P, _P, _P, _P, _I, _P, _I, _I, _P, _P, _I, _I, _I,
                                      _I, _P, _P]),
    "paged_decode_attn_partition_tokens": (ctypes.c_int32, [_I, _I, _I, _I, _I]),
    "paged_decode_attn_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I, _I, _I]),
    "paged_decode_attn": (ctypes.c_int, [_P, _I, _P, _P, _P, _P, _P, _I, _P, _I, _P, _P,
                                         ctypes.c_float, _I, _I, _I, _I, _I, _I, _I, _P,
                                         ctypes.c_size_t, _P]),
    "paged_decode_attn_append": (ctypes.c_int, [_P, _P, _P, _I, _P, _P, _P, _P, _P, _I, _P, _I,
                                                _P, _P, ctypes.c_float, _I, _I, _I, _I, _I, _I,
                                                _I, _P, ctypes.c_size_t, _P]),
    "paged_decode_attn_append_noalloc": (ctypes.c_int, [_P, _P, _P, _I, _P, _P, _P, _P, _P, _I,
                                                        _P, _I, _P, _P, ctypes.c_float, _I, _I,
                                                        _I, _I, _I, _I, _I, _P]),
    "kv_amax_accumulate": (ctypes.c_int, [_P, _L, _I, _I, _P, _P]),
    "wq_packed_bytes": (ctypes.c_size_t, [_I, _I, _I]),
    "wq_quantize_pack": (ctypes.c_int, [_P, _I, _I, _I, _P, _P, _P]),
    "wq_gemv": (ctypes.c_int, [_P, _I, _P, _P, _I, _I, _I, _P, _P]),
    "kv_pool_create": (ctypes.c_int, [_I, _I, ctypes.c_uint32, ctypes.POINTER(_P)]),
    "kv_pool_destroy": (None, [_P]),
    "kv_pool_alloc": (ctypes.c_int, [_P, _I, _P, _P]),
    "kv_pool_free": (ctypes.c_int, [_P, _P, _I]),
    "kv_pool_tags": (ctypes.c_int, [_P, _P]),
    "kv_pool_record_check": (ctypes.c_int, [_P, _P, _I]),
    "kv_pool_get_stats": (ctypes.c_int, [_P, _P]),
    "kv_scales_from_amax": (ctypes.c_int, [_P, _I, _P, _P]),
    "kv_ingest_prefill": (ctypes.c_int, [_P, _P, _L, _P, _P, _I, _I, _P, _I, _I, _P, _P, _P, _P,
                                         _I, _I, _I, _I, _P, _P]),
}


def load():
    """Load libkvfp8.so once and declare the C signatures."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise KvLibraryMissing(
                f"{path} not found; build it with `python -m fp8_e4m3_paged_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def kv_status_str(status: int) -> str:
    return load().kv_status_str(int(status)).decode()


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _ptr(t, name, dtypes=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _check(fn, status):
    if status != 0:
        raise KvError(fn, status)


class Prepared:
    """One checked call of a C entry point, with its arguments fixed.

    Calling the object enqueues the same call again, on the stream fixed when
    it was prepared, without re-checking the tensors or rebuilding the
    argument list: a decode loop whose buffers stay in place pays the host-side
    checks once instead of on every layer of every step. The object holds
    references to the tensors it was prepared with, so their memory stays
    valid; their contents (lengths, flags, new tokens) may change between
    calls. A call that the library refuses raises ``KvError``.

    Sizes are fixed with the arguments, ``max_seq_len`` of the attention
    calls included: every later value in ``seq_lens`` must stay at or below
    the ``max_seq_len`` given when the call was prepared. A request whose
    length exceeds it is refused by the kernels like any too-long request
    (all-zero output, and in the fused call its new token is not stored), not
    reported as an error. Prepare with the largest length the loop will reach.
    """

    __slots__ = ("name", "_fn", "_args", "_keep")

    def __init__(self, name, fn, args, keep):
        self.name = name
        self._fn = fn
        # ctypes objects of the declared types: the per-call conversion is then a type check
        self._args = tuple(a if a is None else t(a) for t, a in zip(fn.argtypes, args))
        self._keep = keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            raise KvError(self.name, st)


def _call(name, args, prepare, keep):
    """Run entry point ``name`` now, or, with ``prepare``, return it as a Prepared."""
    fn = getattr(load(), name)
    if prepare:
        return Prepared(name, fn, args, keep)
    _check(name, fn(*args))
    return None


def _tile_bytes(fp8):
    """Bytes of one (page, KV head) tile: 16 tokens x 128 dims of e4m3 or bf16."""
    return PAGE_SIZE * HEAD_DIM * (1 if fp8 else 2)


def _check_pools(k_pool, v_pool, hkv, fp8):
    """The kernels address whole tiles, so each pool must be [num_pages][num_kv_heads]
    followed by exactly one tile per (page, head)."""
    if k_pool.dim() < 2 or tuple(k_pool.shape) != tuple(v_pool.shape) or k_pool.shape[1] != hkv:
        raise ValueError("k_pool / v_pool must be alike, [num_pages][num_kv_heads][...]")
    per = k_pool.element_size()
    for s in k_pool.shape[2:]:
        per *= s
    if per != _tile_bytes(fp8):
        raise ValueError(f"pools must hold {_tile_bytes(fp8)} bytes per (page, KV head), "
                         f"not {per}")


def _check_requests(batch, seq_lens, block_table, abort=None):
    if seq_lens.numel() != batch:
        raise ValueError(f"seq_lens must hold {batch} lengths")
    if block_table.dim() != 2 or block_table.shape[0] != batch:
        raise ValueError(f"block_table must be [{batch}][bt_stride]")
    if abort is not None and abort.numel() != batch:
        raise ValueError(f"abort must hold {batch} flags")


def _check_scales(k_scale, v_scale, hkv, fp8):
    if not fp8:
        return
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        if t is not None and t.numel() != hkv:
            raise ValueError(f"{name} must hold {hkv} scales (one per KV head)")


_DTYPES = None


def _dt():
    """Accepted torch dtypes per argument kind (built once, on first use)."""
    global _DTYPES
    if _DTYPES is None:
        import torch
        _DTYPES = dict(
            i32=(torch.int32,), u32=(torch.int32, torch.uint32), u8=(torch.uint8,),
            bf16=(torch.bfloat16, torch.int16, torch.uint16), f32=(torch.float32,),
            pool=(torch.uint8, torch.int16, torch.bfloat16, torch.uint16),
        )
    return _DTYPES


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def kv_verify_tags_workspace_bytes(batch, bt_stride):
    return int(load().kv_verify_tags_workspace_bytes(batch, bt_stride))


def kv_verify_tags(pool_tags, block_table, expected_tags, seq_lens, abort_out,
                   page_size=PAGE_SIZE, stream=None, prepare=False, workspace=None):
    """abort_out[b] = 1 iff request b's recorded (page, tag) pairs disagree with the pool.
    ``workspace`` (optional, zero-filled once, kv_verify_tags_workspace_bytes long)
    lets several workgroups share a long row. With prepare=True nothing is
    enqueued; the checked call is returned as a ``Prepared``."""
    d = _dt()
    batch = seq_lens.numel()
    if block_table.dim() != 2 or expected_tags.shape != block_table.shape:
        raise ValueError("block_table / expected_tags must be [batch][bt_stride] alike")
    if block_table.shape[0] != batch or abort_out.numel() != batch:
        raise ValueError("batch mismatch")
    args = (_ptr(pool_tags, "pool_tags", d["u32"]), pool_tags.numel(),
            _ptr(block_table, "block_table", d["i32"]),
            _ptr(expected_tags, "expected_tags", d["u32"]),
            block_table.shape[1], _ptr(seq_lens, "seq_lens", d["i32"]),
            batch, page_size, _ptr(abort_out, "abort_out", d["u8"]),
            _ptr(workspace, "workspace", allow_none=True),
            0 if workspace is None else workspace.numel() * workspace.element_size(),
            _stream(stream))
    return _call("kv_verify_tags", args, prepare,
                 (pool_tags, block_table, expected_tags, seq_lens, abort_out, workspace))


def _append(fp8, k_new, v_new, tok_seq, tok_pos, block_table, k_scale, v_scale, k_pool, v_pool,
            abort=None, batch=None, page_size=PAGE_SIZE, stream=None, prepare=False):
    d = _dt()
    n_tok = tok_seq.numel()
    if tok_pos.numel() != n_tok:
        raise ValueError("tok_seq / tok_pos length mismatch")
    if k_new.dim() != 3 or k_new.shape != v_new.shape or k_new.shape[0] != n_tok:
        raise ValueError("k_new / v_new must be [n_tok][num_kv_heads][head_dim]")
    hkv, hd = k_new.shape[1], k_new.shape[2]
    _check_pools(k_pool, v_pool, hkv, fp8)
    num_pages = k_pool.shape[0]
    if block_table.dim() != 2:
        raise ValueError("block_table must be [batch][bt_stride]")
    if batch is None:
        batch = block_table.shape[0]
    if block_table.shape[0] != batch or (abort is not None and abort.numel() != batch):
        raise ValueError(f"block_table rows and abort must match batch {batch}")
    _check_scales(k_scale, v_scale, hkv, fp8)
    keep = (k_new, v_new, tok_seq, tok_pos, block_table, k_scale, v_scale, k_pool, v_pool, abort)
    if fp8:
        args = (
            _ptr(k_new, "k_new", d["bf16"]), _ptr(v_new, "v_new", d["bf16"]),
            _ptr(tok_seq, "tok_seq", d["i32"]), _ptr(tok_pos, "tok_pos", d["i32"]), n_tok,
            _ptr(block_table, "block_table", d["i32"]), block_table.shape[1], batch,
            _ptr(k_scale, "k_scale", d["f32"]), _ptr(v_scale, "v_scale", d["f32"]),
            _ptr(k_pool, "k_pool", d["u8"]), _ptr(v_pool, "v_pool", d["u8"]), num_pages, hkv,
            hd, page_size, _ptr(abort, "abort", d["u8"], allow_none=True), _stream(stream))
        return _call("kv_append_quant", args, prepare, keep)
    args = (
        _ptr(k_new, "k_new", d["bf16"]), _ptr(v_new, "v_new", d["bf16"]),
        _ptr(tok_seq, "tok_seq", d["i32"]), _ptr(tok_pos, "tok_pos", d["i32"]), n_tok,
        _ptr(block_table, "block_table", d["i32"]), block_table.shape[1], batch,
        _ptr(k_pool, "k_pool", d["pool"]), _ptr(v_pool, "v_pool", d["pool"]), num_pages,
        hkv, hd, page_size, _ptr(abort, "abort", d["u8"], allow_none=True), _stream(stream))
    return _call("kv_append_bf16", args, prepare, keep)


def kv_append_quant(k_new, v_new, tok_seq, tok_pos, block_table, k_scale, v_scale, k_pool,
                    v_pool, abort=None, batch=None, page_size=PAGE_SIZE, stream=None,
                    prepare=False):
    """Quantize new K/V rows to E4M3 with per-KV-head scales and write them into pool pages.
    With prepare=True nothing is enqueued; the checked call is returned as a ``Prepared``."""
    return _append(True, k_new, v_new, tok_seq, tok_pos, block_table, k_scale, v_scale, k_pool,
                   v_pool, abort, batch, page_size, stream, prepare)


def kv_append_bf16(k_new, v_new, tok_seq, tok_pos, block_table, k_pool, v_pool, abort=None,
                   batch=None, page_size=PAGE_SIZE, stream=None, prepare=False):
    """Write new bf16 K/V rows unchanged into BF16 pool pages.
    With prepare=True nothing is enqueued; the checked call is returned as a ``Prepared``."""
    return _append(False, k_new, v_new, tok_seq, tok_pos, block_table, None, None, k_pool,
                   v_pool, abort, batch, page_size, stream, prepare)


def paged_decode_attn_partition_tokens(batch, num_kv_heads, max_seq_len, partition_tokens=0,
                                       cache_dtype=KV_CACHE_FP8_E4M3):
    v = load().paged_decode_attn_partition_tokens(batch, num_kv_heads, max_seq_len,
                                                  partition_tokens, int(cache_dtype))
    if v < 0:
        raise KvError("paged_decode_attn_partition_tokens", v)
    return v


def paged_decode_attn_workspace_bytes(batch, num_q_heads, num_kv_heads, max_seq_len,
                                      partition_tokens=0, head_dim=HEAD_DIM,
                                      cache_dtype=KV_CACHE_FP8_E4M3):
    return int(load().paged_decode_attn_workspace_bytes(batch, num_q_heads, num_kv_heads,
                                                        head_dim, max_seq_len,
                                                        partition_tokens, int(cache_dtype)))


def paged_decode_attn(q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens, max_seq_len,
                      out, sm_scale, workspace=None, abort=None, partition_tokens=0,
                      cache_dtype=KV_CACHE_FP8_E4M3, page_size=PAGE_SIZE, stream=None,
                      prepare=False):
    """out[b][h] = softmax attention of q[b][h] over request b's cached tokens.
    A request longer than max_seq_len outputs zeros. With prepare=True nothing
    is enqueued; the checked call is returned as a ``Prepared``, whose later
    seq_lens must stay <= this max_seq_len."""
    d = _dt()
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q / out must both be [batch][num_q_heads][head_dim]")
    batch, hq, hd = q.shape
    hkv = k_pool.shape[1]
    fp8 = cache_dtype == KV_CACHE_FP8_E4M3
    _check_pools(k_pool, v_pool, hkv, fp8)
    _check_requests(batch, seq_lens, block_table, abort)
    _check_scales(k_scale, v_scale, hkv, fp8)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _ptr(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    args = (
        _ptr(q, "q", d["bf16"]), int(cache_dtype),
        _ptr(k_pool, "k_pool", d["u8"] if fp8 else d["pool"]),
        _ptr(v_pool, "v_pool", d["u8"] if fp8 else d["pool"]),
        _ptr(k_scale, "k_scale", d["f32"], allow_none=not fp8),
        _ptr(v_scale, "v_scale", d["f32"], allow_none=not fp8),
        _ptr(block_table, "block_table", d["i32"]), block_table.shape[1],
        _ptr(seq_lens, "seq_lens", d["i32"]), int(max_seq_len),
        _ptr(abort, "abort", d["u8"], allow_none=True), _ptr(out, "out", d["f32"]),
        float(sm_scale), batch, hq, hkv, hd, page_size, k_pool.shape[0], int(partition_tokens),
        ws_ptr, ws_bytes, _stream(stream))
    return _call("paged_decode_attn", args, prepare,
                 (q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens, abort, out,
                  workspace))


def paged_decode_attn_append(q, k_new, v_new, k_pool, v_pool, k_scale, v_scale, block_table,
                             seq_lens, max_seq_len, out, sm_scale, workspace=None, abort=None,
                             partition_tokens=0, cache_dtype=KV_CACHE_FP8_E4M3,
                             page_size=PAGE_SIZE, stream=None, prepare=False):
    """Append each request's new token (position seq_lens[b] - 1) and attend, in one launch.
    A request longer than max_seq_len is neither written nor read (zeros). With
    prepare=True nothing is enqueued; the checked call is returned as a
    ``Prepared``, whose later seq_lens must stay <= this max_seq_len."""
    d = _dt()
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q / out must both be [batch][num_q_heads][head_dim]")
    batch, hq, hd = q.shape
    hkv = k_pool.shape[1]
    if k_new.shape != (batch, hkv, hd) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [batch][num_kv_heads][head_dim]")
    fp8 = cache_dtype == KV_CACHE_FP8_E4M3
    _check_pools(k_pool, v_pool, hkv, fp8)
    _check_requests(batch, seq_lens, block_table, abort)
    _check_scales(k_scale, v_scale, hkv, fp8)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _ptr(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    args = (
        _ptr(q, "q", d["bf16"]), _ptr(k_new, "k_new", d["bf16"]), _ptr(v_new, "v_new", d["bf16"]),
        int(cache_dtype), _ptr(k_pool, "k_pool", d["u8"] if fp8 else d["pool"]),
        _ptr(v_pool, "v_pool", d["u8"] if fp8 else d["pool"]),
        _ptr(k_scale, "k_scale", d["f32"], allow_none=not fp8),
        _ptr(v_scale, "v_scale", d["f32"], allow_none=not fp8),
        _ptr(block_table, "block_table", d["i32"]), block_table.shape[1],
        _ptr(seq_lens, "seq_lens", d["i32"]), int(max_seq_len),
        _ptr(abort, "abort", d["u8"], allow_none=True), _ptr(out, "out", d["f32"]),
        float(sm_scale), batch, hq, hkv, hd, page_size, k_pool.shape[0], int(partition_tokens),
        ws_ptr, ws_bytes, _stream(stream))
    return _call("paged_decode_attn_append", args, prepare,
                 (q, k_new, v_new, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens,
                  abort, out, workspace))


def paged_decode_attn_append_noalloc(q, k_new, v_new, k_pool, v_pool, k_scale, v_scale,
                                     block_table, seq_lens, max_seq_len, out, sm_scale,
                                     abort=None, partition_tokens=0,
                                     cache_dtype=KV_CACHE_FP8_E4M3, page_size=PAGE_SIZE,
                                     stream=None, prepare=False):
    """paged_decode_attn_append with the library's own static split-K scratch
    (KV_NOALLOC_SCRATCH_BYTES per GPU) instead of a workspace argument: the C
    call allocates nothing. Calls that overlap on one GPU race on the scratch."""
    d = _dt()
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q / out must both be [batch][num_q_heads][head_dim]")
    batch, hq, hd = q.shape
    hkv = k_pool.shape[1]
    if k_new.shape != (batch, hkv, hd) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [batch][num_kv_heads][head_dim]")
    fp8 = cache_dtype == KV_CACHE_FP8_E4M3
    _check_pools(k_pool, v_pool, hkv, fp8)
    _check_requests(batch, seq_lens, block_table, abort)
    _check_scales(k_scale, v_scale, hkv, fp8)
    args = (
        _ptr(q, "q", d["bf16"]), _ptr(k_new, "k_new", d["bf16"]), _ptr(v_new, "v_new", d["bf16"]),
        int(cache_dtype), _ptr(k_pool, "k_pool", d["u8"] if fp8 else d["pool"]),
        _ptr(v_pool, "v_pool", d["u8"] if fp8 else d["pool"]),
        _ptr(k_scale, "k_scale", d["f32"], allow_none=not fp8),
        _ptr(v_scale, "v_scale", d["f32"], allow_none=not fp8),
        _ptr(block_table, "block_table", d["i32"]), block_table.shape[1],
        _ptr(seq_lens, "seq_lens", d["i32"]), int(max_seq_len),
        _ptr(abort, "abort", d["u8"], allow_none=True), _ptr(out, "out", d["f32"]),
        float(sm_scale), batch, hq, hkv, hd, page_size, k_pool.shape[0], int(partition_tokens),
        _stream(stream))
    return _call("paged_decode_attn_append_noalloc", args, prepare,
                 (q, k_new, v_new, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens,
                  abort, out))


def decode_step(layers, block_table, seq_lens, tok_pos, tok_seq, max_seq_len, sm_scale,
                pool_tags=None, expected_tags=None, abort=None, cache_dtype=KV_CACHE_FP8_E4M3,
                workspace=None, partition_tokens=0, fused=True, stream=None,
                verify_workspace=None):
    """Enqueue one decode step: tag check (if pool_tags is given), then for
    each layer the append of the new token and attention over the pages
    (one fused launch per layer, or the two separate calls with fused=False).

    ``layers`` is a sequence of dicts with keys q, k_new, v_new, k_pool, v_pool,
    k_scale, v_scale, out. With pool_tags=None no check runs and abort=None is
    passed on (the no-op tracker). ``verify_workspace`` goes to the tag check.
    """
    if pool_tags is not None:
        kv_verify_tags(pool_tags, block_table, expected_tags, seq_lens, abort, stream=stream,
                       workspace=verify_workspace)
    else:
        abort = None
    for ly in layers:
        if fused:
            paged_decode_attn_append(ly["q"], ly["k_new"], ly["v_new"], ly["k_pool"],
                                     ly["v_pool"], ly.get("k_scale"), ly.get("v_scale"),
                                     block_table, seq_lens, max_seq_len, ly["out"], sm_scale,
                                     workspace=workspace, abort=abort,
                                     partition_tokens=partition_tokens, cache_dtype=cache_dtype,
                                     stream=stream)
            continue
        if cache_dtype == KV_CACHE_FP8_E4M3:
            kv_append_quant(ly["k_new"], ly["v_new"], tok_seq, tok_pos, block_table,
                            ly["k_scale"], ly["v_scale"], ly["k_pool"], ly["v_pool"],
                            abort=abort, stream=stream)
        else:
            kv_append_bf16(ly["k_new"], ly["v_new"], tok_seq, tok_pos, block_table,
                           ly["k_pool"], ly["v_pool"], abort=abort, stream=stream)
        paged_decode_attn(ly["q"], ly["k_pool"], ly["v_pool"], ly.get("k_scale"),
                          ly.get("v_scale"), block_table, seq_lens, max_seq_len, ly["out"],
                          sm_scale, workspace=workspace, abort=abort,
                          partition_tokens=partition_tokens, cache_dtype=cache_dtype,
                          stream=stream)


def kv_amax_accumulate(x, amax_inout, stream=None):
    """amax_inout[g] = max(amax_inout[g], max |x[:, g, :]|) over the finite bf16 values."""
    d = _dt()
    if x.dim() != 3 or amax_inout.numel() != x.shape[1]:
        raise ValueError("x must be [rows][num_kv_heads][head_dim], amax_inout [num_kv_heads]")
    st = load().kv_amax_accumulate(_ptr(x, "x", d["bf16"]), x.shape[0], x.shape[1], x.shape[2],
                                   _ptr(amax_inout, "amax_inout", d["f32"]), _stream(stream))
    _check("kv_amax_accumulate", st)


def kv_scales_from_amax(amax, scale_out, stream=None):
    """scale_out = max(fp32(amax / 448), FLT_MIN) for finite amax > 0, else 1.0."""
    d = _dt()
    if scale_out.numel() != amax.numel():
        raise ValueError("amax / scale_out size mismatch")
    st = load().kv_scales_from_amax(_ptr(amax, "amax", d["f32"]), amax.numel(),
                                    _ptr(scale_out, "scale_out", d["f32"]), _stream(stream))
    _check("kv_scales_from_amax", st)


def kv_ingest_prefill(k_rows, v_rows, row_start, seq_lens, block_table, k_pool, v_pool,
                      max_seq_len, k_scale=None, v_scale=None, abort=None,
                      cache_dtype=KV_CACHE_FP8_E4M3, page_size=PAGE_SIZE, stream=None):
    """Write whole prompts (row_start[b] .. + seq_lens[b] of k_rows / v_rows) into their pages."""
    d = _dt()
    if k_rows.dim() != 3 or v_rows.shape != k_rows.shape:
        raise ValueError("k_rows / v_rows must be [rows][num_kv_heads][head_dim]")
    n_rows, hkv, hd = k_rows.shape
    fp8 = cache_dtype == KV_CACHE_FP8_E4M3
    _check_pools(k_pool, v_pool, hkv, fp8)
    batch = seq_lens.numel()
    if row_start.numel() != batch:
        raise ValueError("row_start must hold one row index per request")
    _check_requests(batch, seq_lens, block_table, abort)
    _check_scales(k_scale, v_scale, hkv, fp8)
    st = load().kv_ingest_prefill(
        _ptr(k_rows, "k_rows", d["bf16"]), _ptr(v_rows, "v_rows", d["bf16"]), n_rows,
        _ptr(row_start, "row_start", d["i32"]), _ptr(seq_lens, "seq_lens", d["i32"]), batch,
        int(max_seq_len), _ptr(block_table, "block_table", d["i32"]), block_table.shape[1],
        int(cache_dtype), _ptr(k_scale, "k_scale", d["f32"], allow_none=not fp8),
        _ptr(v_scale, "v_scale", d["f32"], allow_none=not fp8),
        _ptr(k_pool, "k_pool", d["u8"] if fp8 else d["pool"]),
        _ptr(v_pool, "v_pool", d["u8"] if fp8 else d["pool"]), k_pool.shape[0], hkv, hd,
        page_size, _ptr(abort, "abort", d["u8"], allow_none=True), _stream(stream))
    _check("kv_ingest_prefill", st)


def ingest_layer(k_rows, v_rows, row_start, seq_lens, block_table, k_pool, v_pool, max_seq_len,
                 k_scale=None, v_scale=None, amax=None, abort=None,
                 cache_dtype=KV_CACHE_FP8_E4M3, stream=None):
    """Prefill handoff of one layer: for FP8, calibrate k_scale / v_scale
    (fp32 [num_kv_heads], written) from the rows' amax, then write the prompts.
    ``amax`` is an optional fp32 [2][num_kv_heads] scratch tensor (zeroed here).
    Everything, the scratch's allocation and zeroing included, is enqueued on
    ``stream`` (a torch stream, a raw HIP stream handle, or None for torch's
    current stream), so the zeroing is ordered before the accumulation."""
    if cache_dtype == KV_CACHE_FP8_E4M3:
        import torch
        hkv = k_rows.shape[1]
        if stream is None or isinstance(stream, torch.cuda.Stream):
            ts = stream if stream is not None else torch.cuda.current_stream(k_rows.device)
        else:
            ts = torch.cuda.ExternalStream(int(getattr(stream, "cuda_stream", stream)),
                                           device=k_rows.device)
        with torch.cuda.stream(ts):
            if amax is None:
                amax = torch.zeros((2, hkv), dtype=torch.float32, device=k_rows.device)
            else:
                amax.zero_()
            kv_amax_accumulate(k_rows, amax[0], stream=ts)
            kv_amax_accumulate(v_rows, amax[1], stream=ts)
            kv_scales_from_amax(amax[0], k_scale, stream=ts)
            kv_scales_from_amax(amax[1], v_scale, stream=ts)
    kv_ingest_prefill(k_rows, v_rows, row_start, seq_lens, block_table, k_pool, v_pool,
                      max_seq_len, k_scale, v_scale, abort=abort, cache_dtype=cache_dtype,
                      stream=stream)


class _PoolStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "num_pages", "free_pages", "pages_allocated", "pages_freed", "checks",
        "requests_checked", "requests_aborted")]


class PagePool:
    """Host page pool and tag tracker (include/kvpool.h). ``tracked=False`` is
    the no-op tracker: tags stay 0 and recorded checks count nothing.

    Arrays are numpy (host memory); ``tags()`` returns the uint32 tag of every
    page, ready to be copied into the device pool_tags that kv_verify_tags reads.
    """

    def __init__(self, num_pages: int, tracked: bool = True, seed: int = 0):
        self._lib = load()
        h = _P()
        _check("kv_pool_create", self._lib.kv_pool_create(int(num_pages), int(bool(tracked)),
                                                          int(seed) & 0xFFFFFFFF, ctypes.byref(h)))
        self._h = h
        self.num_pages = int(num_pages)
        self.tracked = bool(tracked)

    def close(self):
        if getattr(self, "_h", None):
            self._lib.kv_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def alloc(self, n: int):
        """n free pages (LIFO) -> (page ids int32[n], their tags uint32[n])."""
        import numpy as np
        pages = np.empty(max(int(n), 0), np.int32)      # n < 0 is refused by the library
        tags = np.empty(max(int(n), 0), np.uint32)
        _check("kv_pool_alloc", self._lib.kv_pool_alloc(self._h, int(n), pages.ctypes.data,
                                                        tags.ctypes.data))
        return pages, tags

    def free(self, pages):
        """Return pages to the pool; each one's tag is bumped (tracked pools)."""
        import numpy as np
        p = np.ascontiguousarray(pages, dtype=np.int32)
        _check("kv_pool_free", self._lib.kv_pool_free(self._h, p.ctypes.data, p.size))

    def tags(self):
        import numpy as np
        t = np.empty(self.num_pages, np.uint32)
        _check("kv_pool_tags", self._lib.kv_pool_tags(self._h, t.ctypes.data))
        return t

    def record_check(self, abort):
        """Count one tag check's outcome (abort flags on the host)."""
        import numpy as np
        a = np.ascontiguousarray(abort, dtype=np.uint8)
        _check("kv_pool_record_check", self._lib.kv_pool_record_check(self._h, a.ctypes.data,
                                                                      a.size))

    def stats(self) -> dict:
        st = _PoolStats()
        _check("kv_pool_get_stats", self._lib.kv_pool_get_stats(self._h, ctypes.byref(st)))
        d = {n: getattr(st, n) for n, _ in _PoolStats._fields_}
        d["mismatch_rate"] = (d["requests_aborted"] / d["requests_checked"]
                              if d["requests_checked"] else 0.0)
        return d


def wq_packed_bytes(n, k, fmt=WQ_INT4):
    return int(load().wq_packed_bytes(int(n), int(k), int(fmt)))


def wq_quantize_pack(w, packed, scales, fmt=WQ_INT4, stream=None):
    """Quantize bf16 weights w [n][k] into packed codes (uint8, wq_packed_bytes)
    and fp32 scales [n / 16][k / 128][16] (layouts in include/kvfp8.h)."""
    d = _dt()
    if w.dim() != 2:
        raise ValueError("w must be [n][k]")
    n, k = w.shape
    if packed.numel() * packed.element_size() < wq_packed_bytes(n, k, fmt):
        raise ValueError("packed buffer too small")
    if scales.numel() != n * (k // 128):
        raise ValueError("scales must hold n * k / 128 floats")
    st = load().wq_quantize_pack(_ptr(w, "w", d["bf16"]), n, k, int(fmt), _ptr(packed, "packed"),
                                 _ptr(scales, "scales", d["f32"]), _stream(stream))
    _check("wq_quantize_pack", st)


def wq_gemv(x, packed, scales, y, n, fmt=WQ_INT4, stream=None):
    """y[m][n] += x[m] . dequant(W)[n] (y fp32 [m][n] holds zeros or a bias)."""
    d = _dt()
    if x.dim() != 2 or y.dim() != 2 or y.shape[0] != x.shape[0] or y.shape[1] != n:
        raise ValueError("x must be [m][k] and y [m][n]")
    m, k = x.shape
    if packed.numel() * packed.element_size() < wq_packed_bytes(n, k, fmt):
        raise ValueError("packed buffer smaller than the codes of an n x k matrix")
    if scales.numel() != n * (k // 128):
        raise ValueError("scales must hold n * k / 128 floats")
    st = load().wq_gemv(_ptr(x, "x", d["bf16"]), m, _ptr(packed, "packed"),
                        _ptr(scales, "scales", d["f32"]), int(n), k, int(fmt),
                        _ptr(y, "y", d["f32"]), _stream(stream))
    _check("wq_gemv", st)
