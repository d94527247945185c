#!/usr/bin/env python3
"""Benchmark of the paged FP8-e4m3 KV-cache decode step on one MI355X.

A step is one pass of the whole hot path over one batch: the batched page-tag
check, then for each layer the quantize-on-append of every request's new
token and split-K paged decode attention (dequantize on read, online softmax,
cross-partition reduction). Inputs are seeded synthetic tensors already
resident in HBM when the timed region starts.

Default workload (the headline point): batch 64, contexts 8192 + U{0..1000}
tokens, 64 query / 8 KV heads, head_dim 128, page 16, 8 layers each with its
own pool, FP8 e4m3 cache, tag check on every step.

Prints ONE JSON line. ``value`` is the algorithmic HBM throughput of the
whole step in GB/s; ``seq_steps_per_s`` is batch * steps / time. The
``roofline`` object is the attention launches timed with HIP events on
their launch stream in a pass of their own; ``cpu_baseline`` is the CPU oracle timed on a bounded
sample of the same workload on this host.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth

# HBM bytes per attention launch of the headline workload from two rocprofv3
# --pmc runs (FETCH_SIZE, WRITE_SIZE), each scaled by what the same counter
# reads for a plain 1 GiB device copy (fetch x2.000, write x1.000); valid only
# for the kernel sources they were taken on (sha256 prefix of decode_attn.hip
# + kv_device.h + kv_launch.h). See profiles/attn_partition_kernel_batch64_ctx8k_hbm_counters.md.
COUNTER_TRAFFIC = {
    "source_sha": "7563e0198cdbc69e",
    "workload": "batch64_ctx8k",
    "read_bytes": 1.14390e9,
    "write_bytes": 2.490e6,
    "algorithmic_bytes": 1143833636,
}


# The same for the prefill page writer (ingest_kernel<FP8>, one layer of the
# headline prompts; profiles/ingest_kernel_batch64_prompts.md) and the INT4 GEMV
# roofline kernel (28672x8192, one token; profiles/wq_gemv_int4_1token.md).
INGEST_COUNTER_TRAFFIC = {
    "sources": ("ingest.hip", "kv_device.h"),
    "source_sha": "adf93a35b9782056",
    "read_bytes": 2.2816e9,
    "write_bytes": 1.1406e9,
}
GEMV_COUNTER_TRAFFIC = {
    "sources": ("gemv.hip", "kv_device.h"),
    "source_sha": "7706fea6e8b160f5",
    "read_bytes": 1.25000e8,
    "write_bytes": 5.734e5,
}


def kernel_source_sha(files=("decode_attn.hip", "kv_device.h", "kv_launch.h")) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "fp8_e4m3_paged_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(entry):
    """Calibrated HBM bytes per launch, or None once the kernel source changed."""
    if kernel_source_sha(entry["sources"]) != entry["source_sha"]:
        return None
    return int(entry["read_bytes"] + entry["write_bytes"])


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; 200 for --config skewed16, whose one-layer "
                         "step is ~0.19 ms)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="batch64", choices=["uniform32", "batch64", "skewed16"])
    ap.add_argument("--cache", default="fp8", choices=["fp8", "bf16"])
    ap.add_argument("--verify", default="on", choices=["on", "off"])
    ap.add_argument("--partition-tokens", type=int, default=-1,
                    help="split-K partition size; -1 = the workload's own (0 = automatic)")
    ap.add_argument("--cpu-baseline", default="on", choices=["on", "off"])
    ap.add_argument("--fused", default="on", choices=["on", "off"],
                    help="append + attention in one launch per layer (paged_decode_attn_append)")
    ap.add_argument("--verify-cost", default="on", choices=["on", "off"],
                    help="also time as many steps with the no-op tracker (no tag check)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time for the oracle sample")
    ap.add_argument("--graph", default="off", choices=["on", "off"],
                    help="step and sweep modes: time the steps as captured HIP graphs (one "
                         "per step, captured before timing) instead of eager launches")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--mode", default="step", choices=["step", "copy", "ingest", "sweep", "gemv"],
                    help="copy: time a plain device copy of --copy-mib MiB (counter "
                         "calibration); ingest: the prefill handoff of one layer's prompts; "
                         "sweep: BF16 vs FP8 decode at 1..64 requests under one pool budget; "
                         "gemv: INT4 vs FP8 weight-only decode GEMV at 1..64 tokens")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--sweep-batches", default=",".join(str(b) for b in SWEEP_BATCHES),
                    help="sweep mode: the request counts to run")
    ap.add_argument("--sweep-caches", default="bf16,fp8", help="sweep mode: the caches to run")
    ap.add_argument("--gemv-tokens", default="1,8,16,32,64",
                    help="--mode gemv: comma-separated token counts (the roofline needs 1)")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 200 if args.mode == "step" and args.config == "skewed16" else 20
    return args


def log(args, msg):
    if not args.quiet:
        print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic bytes (what the method must move), per step
# ---------------------------------------------------------------------------
def step_bytes(wl, seq_lens, cache, verify):
    """Bytes one step must read or write, split by operation."""
    import numpy as np
    B, Hq, Hkv, D, P = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size
    esz = 1 if cache == "fp8" else 2
    L = seq_lens.astype(np.int64)
    pages = -(-L // P)
    kv_read = int(L.sum()) * 2 * Hkv * D * esz                 # K and V of every token
    attn_io = B * Hq * D * 2 + B * Hq * D * 4 + int(pages.sum()) * 4 + B * 4
    append = B * Hkv * D * 2 * 2 + B * Hkv * D * 2 * esz + B * 12
    check = int(pages.sum()) * 12 + B * 5 if verify else 0
    per_layer_attn = kv_read + attn_io
    total = check + wl.num_layers * (per_layer_attn + append)
    return dict(total=total, attn_per_layer=per_layer_attn, kv_per_layer=kv_read,
                append_per_layer=append, check=check)


# ---------------------------------------------------------------------------
# CPU oracle leg (bounded sample)
# ---------------------------------------------------------------------------
def cpu_baseline(args, wl, scales, step_index):
    """Time the oracle's step work (tag check, append, attention) for a few
    requests of layer 0 on this host; scale to sequence-steps per second."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import e4m3, paged

    P = wl.page_size
    ks, vs = scales
    order = np.argsort(wl.seq_lens0)[::-1]          # longest first, then shortest
    sample_reqs = [int(order[0]), int(order[-1]), int(order[len(order) // 2])]
    prepared = []
    for b in sample_reqs:
        L0 = int(wl.seq_lens0[b]) + step_index          # tokens already in the pool
        L = L0 + 1
        n = -(-L // P)
        k = e4m3.quantize(wl.kv_bits(0, "k", b, 0, L0), ks[None, :, None])
        v = e4m3.quantize(wl.kv_bits(0, "v", b, 0, L0), vs[None, :, None])
        kp = np.zeros((n, wl.num_kv_heads, P, wl.head_dim), np.uint8)
        vp = np.zeros_like(kp)
        for j in range(n):
            m = max(0, min(P, L0 - j * P))
            kp[j, :, :m] = k[j * P:j * P + m].transpose(1, 0, 2)
            vp[j, :, :m] = v[j * P:j * P + m].transpose(1, 0, 2)
        bt = np.arange(n, dtype=np.int32)[None, :]
        tags = np.arange(n, dtype=np.uint32)
        q = wl.q_bits(0, step_index)[b:b + 1]
        kn = wl.kv_bits(0, "k", b, L0, L)
        vn = wl.kv_bits(0, "v", b, L0, L)
        prepared.append((b, L, kp, vp, bt, tags, q, kn, vn))
    sm = 1.0 / math.sqrt(wl.head_dim)

    def one_run(r):
        b, L, kp, vp, bt, tags, q, kn, vn = r
        kp2, vp2 = kp.copy(), vp.copy()
        ab = paged.verify_tags(tags, bt, tags[None, :], np.array([L]), P)
        paged.append_fp8(kp2, vp2, kn, vn, np.array([0]), np.array([L - 1]), bt, ks, vs, ab)
        paged.decode_attn(q, kp2, vp2, ks, vs, bt, np.array([L], np.int32), sm, "fp8", ab)

    # one thread per usable core (at most 16: a host's CPU share per GPU), each with BLAS
    # at one thread; numpy releases the GIL in the oracle's array work. Each
    # thread runs the sampled requests in turn for the same wall-clock window.
    try:
        n_threads = len(os.sched_getaffinity(0))
    except AttributeError:
        n_threads = os.cpu_count() or 1
    n_threads = max(1, min(16, n_threads))
    wall = max(2.0, 2.0 * args.cpu_seconds / n_threads)
    tokens = [0] * n_threads
    runs = [0] * n_threads
    start = threading.Barrier(n_threads + 1)
    window = {}
    with threadpool_limits(limits=1):
        def worker(i):
            one_run(prepared[i % len(prepared)])               # untimed: first touch
            start.wait()
            start.wait()                                       # the window is set
            k = i
            while time.perf_counter() < window["stop"]:
                r = prepared[k % len(prepared)]
                one_run(r)
                tokens[i] += r[1]
                runs[i] += 1
                k += 1

        threads = [threading.Thread(target=worker, args=(i,)) for i in range(n_threads)]
        for t in threads:
            t.start()
        start.wait()                                           # every thread warmed up
        t0 = time.perf_counter()
        window["stop"] = t0 + wall
        start.wait()
        for t in threads:
            t.join()
        elapsed = time.perf_counter() - t0
    done = sum(runs)
    tok_per_s = sum(tokens) / elapsed
    # one sequence-step = every layer of one request; scale by mean context
    mean_L = float(wl.seq_lens0.mean()) + step_index + 1
    sec_per_seq_step = wl.num_layers * mean_L / tok_per_s
    return {
        "value": 1.0 / sec_per_seq_step,
        "unit": "seq-steps/s",
        "cores": n_threads,
        "kind": "oracle",
        "sample": (f"{done} oracle (tag check + append + attention) runs of layer 0 for "
                   f"requests {sample_reqs} (lengths {sorted(set(r[1] for r in prepared))}) "
                   f"on {n_threads} threads for {elapsed:.1f} s "
                   f"(~{n_threads * elapsed:.0f} s of CPU; host has {os.cpu_count()} cpus); "
                   f"scaled by {wl.num_layers} layers and mean context {mean_L:.0f}"),
        "effective_GBps": None,
    }


def copy_calibration(args):
    """A plain device-to-device copy of known size: the reference that HBM
    byte counters are scaled by."""
    import torch
    n = args.copy_mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    print(json.dumps({"mode": "copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n,
                      "ms_per_copy": round(ms, 4), "GBps_read_plus_write": round(2 * n / ms / 1e6, 1)}),
          flush=True)


def _per_call_ms(fn, reps):
    """Mean milliseconds of one fn() call: a HIP event pair on the current
    stream around each call, so host-side pauses between calls (which leave
    the GPU idle) are not counted in a per-kernel figure."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / reps


def _back_to_back_ms(fn, reps, per=8):
    """Mean milliseconds of one fn() call within runs of `per` back-to-back
    calls: one untimed call first keeps the GPU busy while the host enqueues
    the run, then one HIP event pair on the current stream spans the run, so
    a short kernel's figure holds neither the event's own dispatch latency
    nor host pauses (kernel-trace durations agree with it)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        fn()
        a.record()
        for _ in range(per):
            fn()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / (reps * per)


def stream_read_peak(reps=10):
    """Streaming-read rate of this GPU through the library's own grid-stride
    read kernel (the prefill amax pass, 16-byte loads, no writes) over 2 GiB:
    the plain-read ceiling the paged kernels can be compared with (the
    roofline fraction itself stays against the published 8 TB/s)."""
    import torch

    import fp8_e4m3_paged_amd as kv
    rows = (2 << 30) // (8 * 128 * 2)
    x = torch.ones((rows, 8, 128), dtype=torch.bfloat16, device="cuda")
    amax = torch.zeros(8, dtype=torch.float32, device="cuda")
    for _ in range(2):
        kv.kv_amax_accumulate(x, amax)
    torch.cuda.synchronize()
    ms = _per_call_ms(lambda: kv.kv_amax_accumulate(x, amax), reps)
    n = x.numel() * 2
    del x
    torch.cuda.empty_cache()
    return {"GBps": round(n / ms / 1e6, 1), "kernel": "amax_kernel (grid-stride 16-byte reads)",
            "bytes": n, "avg_launch_us": round(ms * 1e3, 2)}


def _events_ms(fn, reps):
    """Mean milliseconds of fn() over reps calls, HIP events on the current stream."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def ingest_bench(args):
    """Prefill handoff of layer 0 of a workload's prompts: per-KV-head amax of
    K and V, the scales, and the page-by-page write of every prompt
    (kv_ingest_prefill), timed as one unit; beside it the same tokens through
    the token-granular bulk kv_append_quant, for comparison."""
    import numpy as np
    import torch

    import fp8_e4m3_paged_amd as kv
    import synth
    from synth import device as sd

    kv.load()
    dev = "cuda"
    make = {"uniform32": synth.uniform_32req, "batch64": synth.batch64_ctx8k, "skewed16": synth.skewed_16req}[args.config]
    wl = make(max_steps=1)
    fp8 = args.cache == "fp8"
    hkv, D, P = wl.num_kv_heads, wl.head_dim, wl.page_size
    ones = np.ones(hkv, np.float32)
    st = sd.DeviceState(wl, kv, cache=args.cache, device=dev, layers=[0], fill=False,
                        scales={0: (ones, ones)})
    kr, start = sd.prompt_rows(wl, 0, "k", dev)
    vr, _ = sd.prompt_rows(wl, 0, "v", dev)
    lens0 = torch.from_numpy(wl.seq_lens0.astype(np.int32)).to(dev)
    max_len = int(wl.seq_lens0.max())
    ks = torch.empty(hkv, dtype=torch.float32, device=dev)
    vs = torch.empty_like(ks)
    amax = torch.zeros((2, hkv), dtype=torch.float32, device=dev)
    cd = kv.KV_CACHE_FP8_E4M3 if fp8 else kv.KV_CACHE_BF16
    kp, vp = st.k_pool[0], st.v_pool[0]

    def handoff():
        kv.ingest_layer(kr, vr, start, lens0, st.block_table, kp, vp, max_len, ks, vs,
                        amax=amax, cache_dtype=cd)

    def ingest_only():
        kv.kv_ingest_prefill(kr, vr, start, lens0, st.block_table, kp, vp, max_len, ks, vs,
                             cache_dtype=cd)

    def amax_only():
        kv.kv_amax_accumulate(kr, amax[0])

    seq = torch.repeat_interleave(torch.arange(wl.batch, dtype=torch.int32, device=dev),
                                  lens0.long()).to(torch.int32)
    pos = torch.cat([torch.arange(int(L), dtype=torch.int32, device=dev)
                     for L in wl.seq_lens0]).to(torch.int32)

    def bulk_append():
        if fp8:
            kv.kv_append_quant(kr, vr, seq, pos, st.block_table, ks, vs, kp, vp)
        else:
            kv.kv_append_bf16(kr, vr, seq, pos, st.block_table, kp, vp)

    for _ in range(max(1, args.warmup)):
        handoff()
    torch.cuda.synchronize()
    reps = max(1, args.steps)
    t_handoff = _events_ms(handoff, reps)
    t_ingest = _per_call_ms(ingest_only, reps)
    t_amax = _per_call_ms(amax_only, reps)
    t_append = _events_ms(bulk_append, max(1, reps // 4))

    n_tok = int(wl.seq_lens0.sum())
    pages = int((-(-wl.seq_lens0.astype(np.int64) // P)).sum())
    esz = 1 if fp8 else 2
    row_bytes = hkv * D * 2                            # one token's bf16 K (or V) row
    tile = P * D * esz
    ingest_bytes = 2 * n_tok * row_bytes + 2 * pages * hkv * tile + wl.batch * 12 + pages * 4
    amax_bytes = 2 * n_tok * row_bytes if fp8 else 0
    total = ingest_bytes + amax_bytes
    append_bytes = 2 * n_tok * row_bytes + 2 * n_tok * hkv * D * esz + n_tok * 8
    res = {
        "metric": "prefill ingest: handoff of one layer's prompts into the paged cache, GB/s",
        "mode": "ingest",
        "value": round(total / t_handoff / 1e6, 1),
        "unit": "GB/s",
        "tokens_per_s": round(n_tok / t_handoff * 1e3, 1),
        "ms_per_layer": round(t_handoff, 4),
        "higher_is_better": True,
        "dtype": "e4m3" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name} prompts, layer 0", "batch": wl.batch,
                   "tokens": n_tok, "pages": pages, "num_kv_heads": hkv, "head_dim": D,
                   "cache": args.cache},
        "roofline": {"bound": "hbm", "kernel": "ingest_kernel (kv_ingest_prefill)",
                     "achieved": round(ingest_bytes / t_ingest / 1e6, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ingest_bytes / t_ingest / 1e6 / HBM_PEAK_GBS, 4),
                     "traffic": (counter_traffic(INGEST_COUNTER_TRAFFIC)
                                 if fp8 and wl.name == "batch64_ctx8k" else None),
                     "avg_launch_us": round(t_ingest * 1e3, 2),
                     "algorithmic_bytes_per_launch": ingest_bytes},
        "amax_kernel": {"GBps": round(2 * n_tok * row_bytes / 2 / t_amax / 1e6, 1),
                        "avg_launch_us": round(t_amax * 1e3, 2)} if fp8 else None,
        "bulk_append_for_comparison": {"GBps": round(append_bytes / t_append / 1e6, 1),
                                       "ms": round(t_append, 4)},
    }
    print(json.dumps(res), flush=True)


SWEEP_BATCHES = (1, 8, 16, 32, 64)


def sweep_bench(args):
    """BF16 vs FP8 cache at 1, 8, 16, 32 and 64 concurrent requests (the
    headline's length draw, 8 layers), under one pool-memory budget: 1.01 x
    the BF16 pools of 32 requests (room for the timed steps included), so
    BF16 runs out above 32 while FP8 reaches 64. Each point that fits runs the
    decode step (tag check, fused append + attention per layer) for --steps
    steps after --warmup, three times over, and reports the median window; a
    point that does not fit is reported as such."""
    import numpy as np
    import torch

    import fp8_e4m3_paged_amd as kv
    import synth
    from synth import device as sd

    kv.load()
    dev = "cuda"
    total_steps = args.warmup + args.steps

    def pool_bytes(wl, cache):
        tile = wl.page_size * wl.head_dim * (1 if cache == "fp8" else 2)
        return wl.num_pages * wl.num_kv_heads * 2 * tile * wl.num_layers

    ref = synth.concurrency_point(32, max_steps=total_steps)
    budget = int(1.01 * pool_bytes(ref, "bf16"))
    points = []
    for cache in args.sweep_caches.split(","):
        for B in [int(x) for x in args.sweep_batches.split(",")]:
            wl = synth.concurrency_point(B, max_steps=total_steps)
            need = pool_bytes(wl, cache)
            pt = {"cache": cache, "batch": B, "pool_GB": round(need / 1e9, 3)}
            if need > budget:
                pt["fits"] = False
                points.append(pt)
                log(args, f"{cache} B={B}: pools need {need / 1e9:.2f} GB > budget")
                continue
            st = sd.DeviceState(wl, kv, cache=cache, device=dev)
            # small points: copies of the 8 layers' pools, one set per step in turn
            # (timing only: a set misses the tokens appended into the others)
            n_sets = max(1, -(-ROTATION_BYTES // need))
            pool_sets = [(st.k_pool, st.v_pool)] + [
                ({l: st.k_pool[l].clone() for l in st.layers},
                 {l: st.v_pool[l].clone() for l in st.layers}) for _ in range(n_sets - 1)]
            pt["pool_copies_rotated"] = n_sets
            seq_lens = [st.seq_lens(i).contiguous() for i in range(total_steps)]
            inputs = [[(sd.q_bits_device(wl, l, i, dev), sd.new_token_bits_device(wl, l, "k", i, dev),
                        sd.new_token_bits_device(wl, l, "v", i, dev))
                       for l in range(wl.num_layers)] for i in range(total_steps)]
            outs = [torch.empty((B, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
                    for _ in range(wl.num_layers)]
            spt = max(args.partition_tokens, 0)          # -1 (default): automatic
            cd = kv.KV_CACHE_FP8_E4M3 if cache == "fp8" else kv.KV_CACHE_BF16
            n = kv.paged_decode_attn_workspace_bytes(B, wl.num_q_heads, wl.num_kv_heads,
                                                     wl.max_seq_len, spt, cache_dtype=cd)
            ws = torch.zeros(max(n, 256), dtype=torch.uint8, device=dev)
            vws_n = kv.kv_verify_tags_workspace_bytes(B, st.block_table.shape[1])
            vws = torch.zeros(vws_n, dtype=torch.uint8, device=dev) if vws_n else None
            sm = 1.0 / math.sqrt(wl.head_dim)

            def step(i, prepare=False):
                kp, vp = pool_sets[i % n_sets]
                calls = [kv.kv_verify_tags(st.pool_tags, st.block_table, st.expected_tags,
                                           seq_lens[i], st.abort, prepare=prepare,
                                           workspace=vws)]
                for l in range(wl.num_layers):
                    q, kn, vn = inputs[i][l]
                    calls.append(kv.paged_decode_attn_append(
                        q, kn, vn, kp[l], vp[l], st.k_scale[l], st.v_scale[l],
                        st.block_table, seq_lens[i], wl.max_seq_len, outs[l], sm, workspace=ws,
                        abort=st.abort, cache_dtype=cd, partition_tokens=spt, prepare=prepare))
                return calls

            for i in range(args.warmup):
                step(i)
            torch.cuda.synchronize()
            # eager: each timed step's calls are checked once here and enqueued from
            # their prepared form (the small points would otherwise time the host's
            # per-call checks); with --graph on, each timed step is replayed from a
            # HIP graph captured here
            graphs = None
            prepared = [step(args.warmup + i, prepare=True) for i in range(args.steps)]
            if args.graph == "on":
                graphs = []
                for i in range(args.steps):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        step(args.warmup + i)
                    graphs.append(g)
                torch.cuda.synchronize()
            # the same K steps timed three times (a step rewrites its own new token,
            # so repeating it is the same work); the median, since the windows of
            # the small points are a few ms and the first can catch the clocks rising
            windows = []
            for _ in range(3):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for i in range(args.steps):
                    if graphs is not None:
                        graphs[i].replay()
                    else:
                        for call in prepared[i]:
                            call()
                b.record()
                torch.cuda.synchronize()
                windows.append(a.elapsed_time(b) / args.steps)
            ms = float(np.median(windows))
            byts = sum(step_bytes(wl, wl.seq_lens_at(args.warmup + i), cache, True)["total"]
                       for i in range(args.steps)) / args.steps
            pt.update(fits=True, ms_per_step=round(ms, 4),
                      seq_steps_per_s=round(B / ms * 1e3, 1), GBps=round(byts / ms / 1e6, 1))
            points.append(pt)
            log(args, f"{cache} B={B}: {ms:.3f} ms/step, {B / ms * 1e3:.0f} seq-steps/s, "
                      f"{byts / ms / 1e6:.0f} GB/s")
            del st, inputs, outs, ws, graphs, prepared, pool_sets
            torch.cuda.empty_cache()
    best = {c: max((p["seq_steps_per_s"] for p in points if p["cache"] == c and p["fits"]),
                   default=None) for c in ("bf16", "fp8")}
    res = {
        "metric": "decode seq-steps/s, BF16 vs FP8 cache, 1..64 requests under one pool budget",
        "mode": "sweep", "value": best["fp8"], "unit": "seq-steps/s", "higher_is_better": True,
        "steps": args.steps, "warmup": args.warmup, "dtype": "e4m3 / bf16", "data": "synthetic",
        "config": {"workload": "headline length draw (8192 + U[0,1000]), first B requests, "
                               "8 layers, 64 q / 8 KV heads, tag check on, fused append",
                   "pool_budget_GB": round(budget / 1e9, 3),
                   "launch": "HIP graph per step" if args.graph == "on"
                             else "eager, calls prepared before timing"},
        "best": best,
        "fp8_over_best_bf16": round(best["fp8"] / best["bf16"], 3) if best["bf16"] else None,
        "points": points,
    }
    print(json.dumps(res), flush=True)


# One decode layer's dense weight stream: (rows n, inputs k) of the attention
# output projection, the fused gate + up projection and the down projection
# of a hidden-8192, FFN-14336 transformer layer.
GEMV_LAYER = ((8192, 8192), (28672, 8192), (8192, 14336))
# MI355X keeps a 256 MB memory-side cache (Infinity Cache) in front of HBM.
# A real model's layers each have their own weights and KV pools, so a
# benchmark whose buffers total less than this cycles through copies of them
# (same contents, distinct buffers) holding at least this many bytes: every
# copy has been evicted by the time it is read again, and each read is an HBM
# read.
ROTATION_BYTES = 768 << 20


def gemv_bench(args):
    """INT4 vs FP8 e4m3 weight-only decode GEMV (wq_gemv) over one layer's
    weight stream at 1, 8, 16, 32 and 64 tokens: time per layer, tokens/s,
    and HBM GB/s of the algorithmic bytes (codes, scales, activations, y)."""
    import numpy as np
    import torch

    import fp8_e4m3_paged_amd as kv

    kv.load()
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    mats, copies = {}, {}
    for fmt in (kv.WQ_INT4, kv.WQ_FP8_E4M3):
        mats[fmt] = []
        for n, k in GEMV_LAYER:
            w = (torch.randn((n, k), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
            packed = torch.empty(kv.wq_packed_bytes(n, k, fmt), dtype=torch.uint8, device=dev)
            scales = torch.empty(n * (k // 128), dtype=torch.float32, device=dev)
            kv.wq_quantize_pack(w, packed, scales, fmt)
            mats[fmt].append((n, k, packed, scales))
            del w
        layer_bytes = sum(p.numel() + s.numel() * 4 for _, _, p, s in mats[fmt])
        n_copies = -(-ROTATION_BYTES // layer_bytes)
        copies[fmt] = [mats[fmt]] + [[(n, k, p.clone(), s.clone()) for n, k, p, s in mats[fmt]]
                                     for _ in range(n_copies - 1)]
    torch.cuda.synchronize()
    points, largest = [], None
    token_counts = [int(t) for t in args.gemv_tokens.split(",")]
    if 1 not in token_counts or any(not 1 <= t <= 4096 for t in token_counts):
        print("--gemv-tokens: counts in 1..4096, including 1", file=sys.stderr)
        sys.exit(2)
    for fmt, name in ((kv.WQ_FP8_E4M3, "fp8"), (kv.WQ_INT4, "int4")):
        for M in token_counts:
            xs = [(torch.randn((M, k), generator=gen, device=dev)).to(torch.bfloat16)
                  for _, k in GEMV_LAYER]
            ys = [torch.zeros((M, n), dtype=torch.float32, device=dev) for n, _ in GEMV_LAYER]

            turn = [0]

            def layer():                                    # the next copy of the layer
                ws = copies[fmt][turn[0] % len(copies[fmt])]
                turn[0] += 1
                for (n, k, packed, scales), x, y in zip(ws, xs, ys):
                    kv.wq_gemv(x, packed, scales, y, n, fmt)

            for _ in range(max(1, args.warmup)):
                layer()
            torch.cuda.synchronize()
            ms = _events_ms(layer, max(1, args.steps))
            byts = sum(p.numel() + s.numel() * 4 + M * k * 2 + 2 * M * n * 4
                       for (n, k, p, s) in mats[fmt])
            points.append({"weights": name, "tokens": M, "us_per_layer": round(ms * 1e3, 2),
                           "tokens_per_s": round(M / ms * 1e3, 1),
                           "GBps": round(byts / ms / 1e6, 1)})
            log(args, f"{name} M={M}: {ms * 1e3:.1f} us/layer, {byts / ms / 1e6:.0f} GB/s")
            if name == "int4" and M == 1:
                n, k, p, s = mats[fmt][1]                 # the largest matrix alone
                x1, y1 = xs[1], ys[1]
                big = [c[1] for c in copies[fmt]]         # its copies, in turn

                def largest_call():
                    _, _, pc, sc = big[turn[0] % len(big)]
                    turn[0] += 1
                    kv.wq_gemv(x1, pc, sc, y1, n, fmt)

                t1 = _back_to_back_ms(largest_call, max(1, args.steps))
                b1 = p.numel() + s.numel() * 4 + k * 2 + 2 * n * 4
                largest = {"bound": "hbm", "kernel": f"wq_gemv_small_kernel<INT4> {n}x{k}, 1 token",
                           "achieved": round(b1 / t1 / 1e6, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(b1 / t1 / 1e6 / HBM_PEAK_GBS, 4),
                           "traffic": counter_traffic(GEMV_COUNTER_TRAFFIC)
                           if (n, k) == (28672, 8192) else None,
                           "avg_launch_us": round(t1 * 1e3, 2),
                           "algorithmic_bytes_per_launch": b1,
                           "weight_copies_rotated": len(big)}
    sp = {M: round(next(p["tokens_per_s"] for p in points if p["weights"] == "int4" and p["tokens"] == M)
                   / next(p["tokens_per_s"] for p in points if p["weights"] == "fp8" and p["tokens"] == M), 3)
          for M in token_counts}
    res = {
        "metric": "weight-only decode GEMV over one layer's weights: tokens/s, INT4 vs FP8",
        "mode": "gemv", "value": next(p["tokens_per_s"] for p in points
                                      if p["weights"] == "int4" and p["tokens"] == 1),
        "unit": "tokens/s", "higher_is_better": True, "dtype": "int4 / e4m3 weights, bf16 x",
        "data": "synthetic", "steps": args.steps, "warmup": args.warmup,
        "config": {"workload": "one layer: " + ", ".join(f"{n}x{k}" for n, k in GEMV_LAYER),
                   "group": 128,
                   "weight_copies": {"int4": len(copies[kv.WQ_INT4]),
                                     "fp8": len(copies[kv.WQ_FP8_E4M3])}},
        "roofline": largest, "int4_over_fp8": sp, "points": points,
    }
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.mode == "copy":
        copy_calibration(args)
        return
    if args.mode in ("ingest", "sweep", "gemv"):
        if args.gpus != 1:
            print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported",
                  file=sys.stderr)
            sys.exit(2)
        {"ingest": ingest_bench, "sweep": sweep_bench, "gemv": gemv_bench}[args.mode](args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library runs on one GPU and has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp8_e4m3_paged_amd as kv
    import synth
    from synth import device as sd

    kv.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    measure_noop = args.verify == "on" and args.verify_cost == "on"
    # timed passes of --steps steps each: the step itself (no per-kernel events,
    # which would add gaps), the attention calls bracketed by events, and
    # optionally the no-op tracker followed by the checked step once more
    total_steps = args.warmup + args.steps * (4 if measure_noop else 2)
    make = {"uniform32": synth.uniform_32req, "batch64": synth.batch64_ctx8k, "skewed16": synth.skewed_16req}[args.config]
    wl = make(max_steps=total_steps)
    pt = wl.partition_tokens if args.partition_tokens < 0 else args.partition_tokens
    verify = args.verify == "on"
    fused = args.fused == "on"
    cache = args.cache
    fp8 = cache == "fp8"
    log(args, f"workload {wl.name}: B={wl.batch} layers={wl.num_layers} pages={wl.num_pages} "
              f"mean L0={wl.seq_lens0.mean():.0f} cache={cache} verify={verify}")

    t0 = time.time()
    st = sd.DeviceState(wl, kv, cache=cache, device=dev)
    torch.cuda.synchronize()
    log(args, f"pools filled in {time.time() - t0:.1f} s")

    # per-step inputs, made on the device before timing
    seq_lens = [st.seq_lens(s).contiguous() for s in range(total_steps)]
    tok_pos = [st.tok_pos(s).contiguous() for s in range(total_steps)]
    inputs = []
    for s in range(total_steps):
        per = []
        for layer in range(wl.num_layers):
            per.append((sd.q_bits_device(wl, layer, s, dev),
                        sd.new_token_bits_device(wl, layer, "k", s, dev),
                        sd.new_token_bits_device(wl, layer, "v", s, dev)))
        inputs.append(per)
    outs = [torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
            for _ in range(wl.num_layers)]
    max_len = wl.max_seq_len
    cd = kv.KV_CACHE_FP8_E4M3 if fp8 else kv.KV_CACHE_BF16
    pt_eff = kv.paged_decode_attn_partition_tokens(wl.batch, wl.num_kv_heads, max_len, pt, cd)
    ws_n = kv.paged_decode_attn_workspace_bytes(wl.batch, wl.num_q_heads, wl.num_kv_heads,
                                                max_len, pt, cache_dtype=cd)
    ws = torch.zeros(max(ws_n, 256), dtype=torch.uint8, device=dev)
    sm = 1.0 / math.sqrt(wl.head_dim)
    stream = torch.cuda.current_stream()

    # fused: one event pair around each step's back-to-back layer launches (the
    # per-launch time is that span over the layer count, so the events' own
    # cost is not counted once per launch); separate calls: a pair per attention call
    ev_attn = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps * (1 if fused else wl.num_layers))]
    # and one pair around each step's tag check, whose time is taken out of the
    # timed pass's step to give the fused launches' share of it
    ev_check = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]

    # counters of the split tag check (rows longer than one 2,048-page chunk)
    vws_n = kv.kv_verify_tags_workspace_bytes(wl.batch, st.block_table.shape[1])
    vws = torch.zeros(vws_n, dtype=torch.uint8, device=dev) if vws_n else None

    def run_step(s, timed_slot=None, check=verify, stream=stream, check_slot=None):
        abort = st.abort if check else None
        if check:
            if check_slot is not None:
                ev_check[check_slot][0].record(stream)
            kv.kv_verify_tags(st.pool_tags, st.block_table, st.expected_tags, seq_lens[s],
                              st.abort, stream=stream, workspace=vws)
            if check_slot is not None:
                ev_check[check_slot][1].record(stream)
        for layer in range(wl.num_layers):
            q, kn, vn = inputs[s][layer]
            if fused:
                if timed_slot is not None and layer == 0:
                    ev_attn[timed_slot][0].record(stream)
                kv.paged_decode_attn_append(q, kn, vn, st.k_pool[layer], st.v_pool[layer],
                                            st.k_scale[layer], st.v_scale[layer], st.block_table,
                                            seq_lens[s], max_len, outs[layer], sm, workspace=ws,
                                            abort=abort, partition_tokens=pt, cache_dtype=cd,
                                            stream=stream)
                if timed_slot is not None and layer == wl.num_layers - 1:
                    ev_attn[timed_slot][1].record(stream)
                continue
            if fp8:
                kv.kv_append_quant(kn, vn, st.tok_seq, tok_pos[s], st.block_table,
                                   st.k_scale[layer], st.v_scale[layer], st.k_pool[layer],
                                   st.v_pool[layer], abort=abort, stream=stream)
            else:
                kv.kv_append_bf16(kn, vn, st.tok_seq, tok_pos[s], st.block_table,
                                  st.k_pool[layer], st.v_pool[layer], abort=abort, stream=stream)
            if timed_slot is not None:
                ev_attn[timed_slot + layer][0].record(stream)
            kv.paged_decode_attn(q, st.k_pool[layer], st.v_pool[layer], st.k_scale[layer],
                                 st.v_scale[layer], st.block_table, seq_lens[s], max_len,
                                 outs[layer], sm, workspace=ws, abort=abort,
                                 partition_tokens=pt, cache_dtype=cd, stream=stream)
            if timed_slot is not None:
                ev_attn[timed_slot + layer][1].record(stream)

    for s in range(args.warmup):
        run_step(s)
    torch.cuda.synchronize()
    log(args, f"warmup done ({args.warmup} steps); timing {args.steps} steps")

    # pass 1: the timed steps (as HIP graphs: one per step, each holding the
    # tag check and the layers' launches with that step's tensors, captured
    # before the timed region; replaying them is the same work with the
    # launch overhead between kernels taken out)
    graphs = None
    if args.graph == "on":
        graphs = []
        for i in range(args.steps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_step(args.warmup + i, stream=torch.cuda.current_stream())
            graphs.append(g)
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        if graphs is not None:
            graphs[i].replay()
        else:
            run_step(args.warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    elapsed_ms = start.elapsed_time(end)
    ms_per_step = elapsed_ms / args.steps
    # checked after the timed pass, so no device-to-host round trip sits
    # between the warm-up and the timed steps
    if verify:
        assert int(st.abort.sum().item()) == 0, "no request of this workload may abort"

    # the same steps timed four more times (the same work again: the appends
    # rewrite the codes they wrote), for the median of five passes beside the
    # first pass, which is what `value` reports
    reps = [elapsed_ms]
    if graphs is None:
        for _ in range(4):
            a_r, b_r = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a_r.record(stream)
            for i in range(args.steps):
                run_step(args.warmup + i)
            b_r.record(stream)
            torch.cuda.synchronize()
            reps.append(a_r.elapsed_time(b_r))
        log(args, f"{len(reps)} passes over the same steps: median "
                  f"{float(np.median(reps)) / args.steps:.4f} ms/step")

    # pass 2: the next steps again with HIP events on the launch stream: around
    # each step's layer launches (fused), or around each attention call
    base2 = args.warmup + args.steps
    torch.cuda.synchronize()
    for i in range(args.steps):
        run_step(base2 + i, timed_slot=i if fused else i * wl.num_layers, check_slot=i)
    torch.cuda.synchronize()
    attn_ms = [a.elapsed_time(b) / (wl.num_layers if fused else 1) for a, b in ev_attn]
    attn_events_ms = float(np.mean(attn_ms))
    # median: a pair of events around one short kernel now and then also holds a
    # stray delay of tens of microseconds
    check_ms = float(np.median([a.elapsed_time(b) for a, b in ev_check])) if verify else 0.0

    by = [step_bytes(wl, wl.seq_lens_at(args.warmup + i), cache, verify)
          for i in range(args.steps)]
    by2 = [step_bytes(wl, wl.seq_lens_at(base2 + i), cache, verify) for i in range(args.steps)]
    total_bytes = sum(b["total"] for b in by)
    gbs = total_bytes / (elapsed_ms * 1e-3) / 1e9
    if fused:
        # the timed pass itself: its step, less the tag check's share, over the
        # back-to-back layer launches (the kernels run with no gap between them)
        attn_avg_ms = (ms_per_step - check_ms) / wl.num_layers
        attn_bytes = float(np.mean([b["attn_per_layer"] + b["append_per_layer"] for b in by]))
    else:
        attn_avg_ms = attn_events_ms
        attn_bytes = float(np.mean([b["attn_per_layer"] for b in by2]))
    attn_gbs = attn_bytes / (attn_avg_ms * 1e-3) / 1e9
    seq_steps = wl.batch * args.steps / (elapsed_ms * 1e-3)
    log(args, f"{ms_per_step:.3f} ms/step, {gbs:.0f} GB/s, attention call {attn_avg_ms*1e3:.1f} us "
              f"= {attn_gbs:.0f} GB/s")

    noop = None
    if measure_noop:
        def timed_pass(base, check):
            """--steps steps from step index `base`, timed the same way as pass 1."""
            a2, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            gs = None
            if args.graph == "on":
                gs = []
                for i in range(args.steps):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        run_step(base + i, check=check, stream=torch.cuda.current_stream())
                    gs.append(g)
            torch.cuda.synchronize()
            a2.record(stream)
            for i in range(args.steps):
                if gs is not None:
                    gs[i].replay()
                else:
                    run_step(base + i, check=check)
            b2.record(stream)
            torch.cuda.synchronize()
            return a2.elapsed_time(b2)

        def kv_bytes(base):
            return sum(step_bytes(wl, wl.seq_lens_at(base + i), cache, False)["kv_per_layer"]
                       for i in range(args.steps))

        # the no-op tracker (no tag check, abort = NULL), then the checked step
        # again, so drift between passes does not favour either: the checked
        # rate is the mean of the passes before and after the no-op one
        base3 = args.warmup + 2 * args.steps
        base4 = args.warmup + 3 * args.steps
        off_ms = timed_pass(base3, False)
        on2_ms = timed_pass(base4, True)
        kv_on = sum(b["kv_per_layer"] for b in by)
        # per KV byte, so the tokens the contexts grew in between do not count
        on_rate = 0.5 * (elapsed_ms / kv_on + on2_ms / kv_bytes(base4))
        overhead = on_rate / (off_ms / kv_bytes(base3)) - 1.0
        noop = {"ms_per_step": round(off_ms / args.steps, 4),
                "checked_after_ms_per_step": round(on2_ms / args.steps, 4),
                "tag_check_overhead_pct": round(100.0 * overhead, 2)}
        log(args, f"no-op tracker: {off_ms / args.steps:.3f} ms/step; tag check costs "
                  f"{100 * overhead:.2f}%")

    cpu = None
    if args.cpu_baseline == "on" and fp8:
        log(args, "timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(args, wl, (st.k_scale_host[0], st.v_scale_host[0]), args.warmup)
        sec_per_seq_step = 1.0 / cpu["value"]
        mean_bytes_per_seq_step = total_bytes / args.steps / wl.batch
        cpu["effective_GBps"] = mean_bytes_per_seq_step / sec_per_seq_step / 1e9

    read_peak = stream_read_peak()
    log(args, f"streaming read through the library's amax pass: {read_peak['GBps']:.0f} GB/s")

    traffic = None
    if (fp8 and wl.name == COUNTER_TRAFFIC["workload"] and pt_eff >= max_len    # one partition
            and kernel_source_sha() == COUNTER_TRAFFIC["source_sha"]):
        traffic = int(COUNTER_TRAFFIC["read_bytes"] + COUNTER_TRAFFIC["write_bytes"])

    result = {
        "metric": "paged FP8-KV decode attn: achieved HBM GB/s + seq-steps/s at B=64, ctx=8k",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "seq_steps_per_s": round(seq_steps, 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median_of_passes": {"passes": len(reps),
                                         "median": round(float(np.median(reps)) / args.steps, 4),
                                         "min": round(min(reps) / args.steps, 4),
                                         "max": round(max(reps) / args.steps, 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3" if fp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"{wl.name}: batch {wl.batch}, ctx 8192+U[0,1000]"
                         if wl.name == "batch64_ctx8k" else wl.name),
            "batch": wl.batch, "layers": wl.num_layers, "num_q_heads": wl.num_q_heads,
            "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
            "page_size": wl.page_size, "mean_ctx": round(float(wl.seq_lens0.mean()) + 1, 1),
            "cache": cache, "verify": verify, "partition_tokens": pt_eff,
            "append": "fused into the attention launch" if fused else "separate launch",
            "launch": "HIP graph per step" if args.graph == "on" else "eager",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("paged_decode_attn_append (append + attention partition kernel)" if fused
                       else "paged_decode_attn (partition kernel + cross-partition reduce)"),
            "achieved": round(attn_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(attn_avg_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": int(attn_bytes),
            "avg_launch_us_events_pass": round(attn_events_ms * 1e3, 2),
            "tag_check_us": round(check_ms * 1e3, 2),
        },
        "cpu_baseline": cpu,
        "no_op_tracker": noop,
        "stream_read_peak": read_peak,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
