#!/usr/bin/env python3
"""Paged decode attention on one MI355X: KV-read GB/s, % of HBM peak and
sequence-tokens per second.

One step is one pa_decode call (one kernel launch) over the whole batch of the
Qwen2.5-7B-shaped workload: 32 sequences, 28 query / 4 KV heads, head_dim 128,
f16 q/K/V, context lengths uniform in [512, 4096], 16-token blocks shuffled
over the pool, split-K pieces merged by log-sum-exp (`--workload` picks one of
the other four for information). Inputs are resident in HBM before timing
starts. Calls rotate over enough copies of the KV pool (>= 3 x 256 MiB) that
the 256 MiB Infinity Cache cannot serve repeats.

Two ways of splitting the work are timed, each over K calls: the workload's
own partitioning (512-token split-K partitions for workloads 3-5, one pass for
1-2) and the balanced split (equal page shares per workgroup, pieces merged by
log-sum-exp); both are reported under "modes". A workload whose sequences
share a prompt prefix also times the shared-prefix call (the balanced split
with the prefix pages read once for all sequences, pa_decode_prefix, mode
"balanced_prefix"). They compute the same result up to float rounding and
meet the same parity bar. `value` is the fastest (--split auto, the default),
or the one --split names.

    python bench.py [--steps K] [--warmup W] [--workload 1..5] [--split auto|spec|balanced|prefix]

Prints one JSON line. `value` is KV-read GB/s: the K and V bytes of every
(sequence, cached token, KV head) the call attends, divided by the time per
call (HIP events on the launching stream around the K timed calls).
`cpu_baseline` times the float64 CPU oracle on the host on the same workload
and checks the GPU output against it.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention KV-read GB/s (% of HBM peak) and seqs·tokens/sec"
PEAK_GBPS = 8000.0            # MI355X HBM3E, published
MALL_BYTES = 256 << 20        # Infinity Cache
CSRC = os.path.join(ROOT, "paged_kv_decode_05_amd", "csrc")
# the sources each kernel is compiled from (its file and the headers it includes)
KERNEL_SRCS = {"decode": ("pa_decode.hip", "pa_tiles.h", "pa_schedule.h", "pa_internal.h"),
               "multi": ("pa_multi.hip", "pa_tiles.h", "pa_internal.h")}
PROBES = os.path.join(ROOT, "tests", "probes", "libpaprobes.so")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--split", choices=["auto", "spec", "balanced", "prefix"], default="auto",
                    help="mode reported as `value`: the faster one, the workload's own "
                         "partition size, the balanced split, or the balanced split with "
                         "the shared prefix read once (workloads with a shared prefix)")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="time only this partition size (0 = one pass, -1 = balanced)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum host time spent timing the oracle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-ceiling", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload record of all five workloads")
    ap.add_argument("--no-flush-check", action="store_true",
                    help="skip the cross-check that times single calls after evicting the caches")
    ap.add_argument("--op", choices=["decode", "multi", "append", "merge", "pool"],
                    default="decode",
                    help="decode: the attention call (default); append: the paged KV "
                         "append of one new token per sequence on the same workload; "
                         "multi: --qlen new tokens per sequence, causal among them "
                         "(pa_decode_multi); "
                         "merge: the log-sum-exp merge of --shards position shards; "
                         "pool: the host block pool's bookkeeping for the workload's "
                         "requests behind a shared prompt prefix")
    ap.add_argument("--shards", type=int, default=8, help="shards for --op merge")
    ap.add_argument("--qlen", type=int, default=8, help="new tokens per sequence for --op multi")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="run a 1 GiB device copy and 20 decode calls, print nothing else "
                         "(for rocprofv3 --pmc counter passes)")
    return ap.parse_args()


def kernel_sha256(kernel="decode"):
    h = hashlib.sha256()
    for name in KERNEL_SRCS[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


# mode value of the shared-prefix call (pa_decode_prefix: the balanced split
# with the workload's shared prefix pages read once for all sequences)
PREFIX = -100


def mode_name(ps):
    return {0: "one_pass", -1: "balanced", PREFIX: "balanced_prefix"}.get(ps, f"partition{ps}")


def mode_partition(ps):
    """The pa_shape partition_size a mode runs with."""
    return -1 if ps == PREFIX else ps


def traffic_from_profile(wl_name, ps, kernel="decode", q_len=None):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    tag = wl_name if q_len is None else f"multi_{wl_name}_T{q_len}"
    path = os.path.join(ROOT, "profiles", f"pmc_traffic_{tag}_{mode_name(ps)}.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            m = re.match(r"^machine:\s*(\{.*\})\s*$", line)
            if m:
                rec = json.loads(m.group(1))
                if rec.get("kernel_sha256") == kernel_sha256(kernel):
                    return rec.get("traffic_bytes_per_launch")
    return None


def stream_read_ceiling(torch):
    """GB/s of a plain streaming-read kernel over 2 GiB on this GPU."""
    import ctypes
    if not os.path.exists(PROBES):
        return None
    lib = ctypes.CDLL(PROBES)
    lib.pa_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_void_p]
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    best = 0.0
    for blocks in (1024, 2048, 4096, 8192):
        for _ in range(2):
            assert lib.pa_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks,
                                            s.cuda_stream) == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        n = 10
        for _ in range(n):
            lib.pa_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks,
                                     s.cuda_stream)
        e1.record(s)
        torch.cuda.synchronize()
        best = max(best, nbytes * n / (e0.elapsed_time(e1) / 1e3) / 1e9)
    del buf
    return best


def blas_threads():
    """Threads the oracle's numpy BLAS may use."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(wl, gpu_out_f64, min_seconds):
    """Time the float64 oracle on the host over the whole workload (repeated
    until min_seconds have passed) and compare the GPU output with it."""
    import numpy as np
    import oracle
    cores = blas_threads()
    s = wl.spec
    reps, t0 = 0, time.perf_counter()
    while True:
        ref = oracle.paged_decode_ref(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                      wl.context_lens, wl.scale, s.io_dtype, s.kv_dtype,
                                      wl.k_scale, wl.v_scale)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    per_call = el / reps
    err = np.abs(gpu_out_f64 - ref)
    return {
        "value": round(wl.kv_bytes_logical() / per_call / 1e9, 4),
        "unit": "GB/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"the whole workload ({s.batch} sequences, "
                  f"{int(wl.context_lens.sum())} cached tokens), {reps} full oracle "
                  f"passes in {el:.1f} s; float64 numpy, BLAS threads = cores",
        "seconds_per_step": round(per_call, 4),
        "parity_vs_gpu": {"max_abs": float(err.max()), "mean_abs": float(err.mean())},
    }


def bench_append(args, torch, np, pkd, W):
    """Time pa_kv_append (one new token per sequence, written at its context
    length) on the workload's shape; bytes = rows read + cache bytes written."""
    import oracle
    spec = W.SPECS[args.workload]
    wl = W.make_workload(spec)
    dev = torch.device("cuda:0")
    t = W.to_device(wl, dev)
    B, H, D = spec.batch, spec.num_kv_heads, spec.head_dim
    src = spec.io_dtype
    rng = np.random.default_rng(1000 + args.workload)
    with np.errstate(over="ignore"):
        k_new = W._to_storage(rng.standard_normal((B, H, D)).astype(np.float32), src)
        v_new = W._to_storage(rng.standard_normal((B, H, D)).astype(np.float32), src)
    pos = np.minimum(wl.context_lens.astype(np.int32), 16 * spec.max_blocks_per_seq - 1)
    kn = W.storage_tensor(k_new, src).to(dev)
    vn = W.storage_tensor(v_new, src).to(dev)
    pt = torch.from_numpy(pos).to(dev)
    pool_bytes = t["k_cache"].numel() * t["k_cache"].element_size() * 2
    reps = max(1, math.ceil(3 * MALL_BYTES / pool_bytes))
    kcs = [t["k_cache"]] + [t["k_cache"].clone() for _ in range(reps - 1)]
    vcs = [t["v_cache"]] + [t["v_cache"].clone() for _ in range(reps - 1)]
    stream = torch.cuda.current_stream()

    from paged_kv_decode_05_amd._lib import prepare_append
    calls = [prepare_append(kn, vn, pt, t["block_table"], kcs[i], vcs[i], k_scale=t["k_scale"],
                            v_scale=t["v_scale"], stream=stream) for i in range(reps)]

    def call(i):
        calls[i % reps]()

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    s_src = oracle.ELEM_BYTES[src]
    s_kv = oracle.ELEM_BYTES[spec.kv_dtype]
    moved = B * H * D * 2 * (s_src + s_kv) + B * 4 * 2
    gbps = moved / (ms / 1e3) / 1e9
    rec = {
        "metric": "paged KV append GB/s (new K/V rows read + cache bytes written)",
        "value": round(gbps, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": src + ("" if spec.kv_dtype == src else "->fp8_e4m3"),
        "data": "synthetic (seeded N(0,1) rows, the workload's block table)",
        "config": {"workload": spec.name, "op": "kv_append", "batch": B, "kv_heads": H,
                   "head_dim": D, "bytes_per_step": moved},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 3), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / PEAK_GBPS, 6), "traffic": None},
        "note": "one token per sequence: a few hundred KB per call, so the call is "
                "launch-latency bound, not bandwidth bound",
    }
    if not args.no_cpu_baseline:
        reps_c, t0 = 0, time.perf_counter()
        while True:
            oracle.kv_append_ref(wl.k_cache, wl.v_cache, k_new, v_new, wl.block_table, pos, src,
                                 spec.kv_dtype, wl.k_scale, wl.v_scale)
            reps_c += 1
            el = time.perf_counter() - t0
            if el >= min(args.cpu_seconds, 5.0):
                break
        rec["cpu_baseline"] = {"value": round(moved / (el / reps_c) / 1e9, 6), "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"the whole call ({B} sequences), {reps_c} oracle passes "
                                         f"in {el:.1f} s (pure Python loop, one thread)"}
    print(json.dumps(rec), flush=True)


def bench_merge(args, torch, np, pkd, W):
    """Time pa_lse_merge of --shards per-shard results on the workload's
    (sequence, query head) rows; bytes = shard outputs and lse read + output
    written."""
    import oracle
    spec = W.SPECS[args.workload]
    B, Hq, D = spec.batch, spec.num_q_heads, spec.head_dim
    S, rows, dt = args.shards, B * Hq, spec.io_dtype
    rng = np.random.default_rng(2000 + args.workload)
    o = W._to_storage(rng.standard_normal((S, rows, D)).astype(np.float32), dt)
    lse = (rng.standard_normal((S, rows)) * 3).astype(np.float32)
    dev = torch.device("cuda:0")
    ot = W.storage_tensor(o, dt).to(dev)
    lt = torch.from_numpy(lse).to(dev)
    out = torch.empty((rows, D), dtype=ot.dtype, device=dev)
    lout = torch.empty(rows, device=dev)
    stream = torch.cuda.current_stream()
    lib = pkd.load_library()
    from paged_kv_decode_05_amd._lib import DTYPE_CODE
    args_c = (S, rows, D, ot.data_ptr(), lt.data_ptr(), DTYPE_CODE[dt], out.data_ptr(),
              lout.data_ptr(), stream.cuda_stream)
    for _ in range(args.warmup):
        assert lib.pa_lse_merge(*args_c) == 0
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        lib.pa_lse_merge(*args_c)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    es = oracle.ELEM_BYTES[dt]
    moved = S * rows * (D * es + 4) + rows * (D * es + 4)
    gbps = moved / (ms / 1e3) / 1e9
    rec = {
        "metric": "log-sum-exp shard merge GB/s (shard outputs + lse read, output written)",
        "value": round(gbps, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic (seeded N(0,1) shard outputs, N(0,9) lse)",
        "config": {"workload": spec.name, "op": "lse_merge", "shards": S, "rows": rows,
                   "head_dim": D, "bytes_per_step": moved},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 3), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / PEAK_GBPS, 6), "traffic": None},
        "note": "decode-sized rows: under 1 MB per call, so the call is launch-latency bound",
    }
    if not args.no_cpu_baseline:
        reps_c, t0 = 0, time.perf_counter()
        while True:
            oracle.shard_merge_ref(o, lse, dt)
            reps_c += 1
            el = time.perf_counter() - t0
            if el >= min(args.cpu_seconds, 5.0):
                break
        rec["cpu_baseline"] = {"value": round(moved / (el / reps_c) / 1e9, 6), "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"the whole call, {reps_c} oracle passes in {el:.1f} s"}
    print(json.dumps(rec), flush=True)


def bench_multi(args, torch, np, pkd, W):
    """Time pa_decode_multi with --qlen new tokens per sequence on the
    workload (their K/V counted in the context lengths, as after the append).
    Bytes = the K/V of every attended (sequence, cached token, KV head), as
    for decode, plus q read and out written; flops = 4 * D per visible
    (query row, key) pair. Both the workload's partition size and the one-pass
    split are timed; `value` is the faster."""
    import oracle
    spec = W.SPECS[args.workload]
    T = args.qlen
    wl = W.make_workload(spec)
    q = W.multi_query(wl, T)
    dev = torch.device("cuda:0")
    t = W.to_device(wl, dev)
    qt = W.storage_tensor(q, spec.io_dtype).to(dev)
    pool_bytes = t["k_cache"].numel() * t["k_cache"].element_size() * 2
    reps = max(1, math.ceil(3 * MALL_BYTES / pool_bytes))
    kcs = [t["k_cache"]] + [t["k_cache"].clone() for _ in range(reps - 1)]
    vcs = [t["v_cache"]] + [t["v_cache"].clone() for _ in range(reps - 1)]
    out = torch.empty_like(qt)
    stream = torch.cuda.current_stream()

    def make_calls(ps):
        ws = None
        if ps:
            ws = torch.empty(pkd.workspace_bytes(qt, t["k_cache"], t["block_table"], ps),
                             dtype=torch.uint8, device=dev)
            pkd.reset_workspace(ws)
        return [pkd.prepare(qt, kcs[i], vcs[i], t["block_table"], t["context_lens"],
                            float(wl.scale), k_scale=t["k_scale"], v_scale=t["v_scale"],
                            partition_size=ps, out=out, workspace=ws, stream=stream)
                for i in range(reps)]

    # the workload's own split, one pass, longer partitions (fewer partial
    # results to write and merge when every row costs a partial) and the
    # balanced split (equal pages per CU: the decode kernels when the rows fit
    # one tile, the wide-row balanced kernel otherwise); the caller picks
    # partition_size
    modes = [args.partition_size] if args.partition_size is not None else \
        [spec.partition_size, 0, 1024, 2048, pkd.SPLIT_BALANCED]
    if args.pmc_pass:
        calls = make_calls(modes[0])
        src = torch.ones(1 << 28, dtype=torch.int32, device=dev)      # 1 GiB
        torch.empty_like(src).copy_(src)
        for i in range(20):
            calls[i % reps]()
        torch.cuda.synchronize()
        return
    timed = {}
    for mode in modes:
        calls = make_calls(mode)
        for i in range(args.warmup):
            calls[i % reps]()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            calls[i % reps]()
        e1.record(stream)
        torch.cuda.synchronize()
        timed[mode] = (e0.elapsed_time(e1) / args.steps,
                       out.float().cpu().numpy().astype(np.float64))
    ps = min(timed, key=lambda m: timed[m][0])
    ms, gpu_out = timed[ps]
    es = oracle.ELEM_BYTES[spec.io_dtype]
    qo_bytes = 2 * spec.batch * T * spec.num_q_heads * spec.head_dim * es
    moved = wl.kv_bytes_logical() + qo_bytes
    L = wl.context_lens.astype(np.int64)
    visible = int(sum(max(int(l) - T + i + 1, 0) for l in L for i in range(T)))
    flops = 4 * spec.head_dim * spec.num_q_heads * visible
    gbps = moved / (ms / 1e3) / 1e9
    tflops = flops / (ms / 1e3) / 1e12
    mfma_peak = {"f32": 157.3, "f16": 2500.0, "bf16": 2500.0}[spec.io_dtype]
    rec = {
        "metric": "multi-token paged attention bytes moved GB/s (KV read + q/out)",
        "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": spec.io_dtype + ("" if spec.kv_dtype == spec.io_dtype else "+fp8_e4m3_kv"),
        "data": "synthetic (seeded N(0,1) q/K/V, seeded lengths and block permutation)",
        "config": {"workload": spec.name, "op": "decode_multi", "q_len": T,
                   "batch": spec.batch, "q_heads": spec.num_q_heads,
                   "kv_heads": spec.num_kv_heads, "head_dim": spec.head_dim,
                   "split": mode_name(ps), "bytes_per_step": moved,
                   "kv_bytes_per_step": wl.kv_bytes_logical(), "flops_per_step": flops,
                   "pool_copies_rotated": reps},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / PEAK_GBPS, 4),
                     "traffic": traffic_from_profile(spec.name, ps, "multi", T)},
        "mfma": {"achieved_TFLOPs": round(tflops, 2), "peak_TFLOPs": mfma_peak,
                 "frac": round(tflops / mfma_peak, 4)},
        "modes": {mode_name(m): {"ms_per_step": round(v[0], 6),
                                 "GBps": round(moved / (v[0] / 1e3) / 1e9, 2)}
                  for m, v in timed.items()},
    }
    if not args.no_cpu_baseline:
        # oracle on whole sequences, in order, until --cpu-seconds pass
        seqs, t0, kvb = [], time.perf_counter(), 0
        per_tok = 2 * spec.num_kv_heads * spec.head_dim * oracle.ELEM_BYTES[spec.kv_dtype]
        while len(seqs) < spec.batch and time.perf_counter() - t0 < args.cpu_seconds:
            b = len(seqs)
            oracle.multi_query_ref(q, wl.k_cache, wl.v_cache, wl.block_table,
                                   wl.context_lens, wl.scale, spec.io_dtype, spec.kv_dtype,
                                   wl.k_scale, wl.v_scale, seqs=[b])
            seqs.append(b)
            kvb += int(L[b]) * per_tok
        el = time.perf_counter() - t0
        ref = oracle.multi_query_ref(q, wl.k_cache, wl.v_cache, wl.block_table,
                                     wl.context_lens, wl.scale, spec.io_dtype, spec.kv_dtype,
                                     wl.k_scale, wl.v_scale, seqs=seqs[:2])
        err = np.abs(gpu_out[seqs[:2]] - ref[seqs[:2]])
        rec["cpu_baseline"] = {"value": round(kvb / el / 1e9, 5), "unit": "GB/s",
                               "cores": int(blas_threads()),
                               "kind": "oracle",
                               "sample": f"{len(seqs)} of {spec.batch} sequences in {el:.1f} s "
                                         f"(KV bytes of those sequences / time)",
                               "parity_vs_gpu": {"max_abs": float(err.max())}}
    print(json.dumps(rec), flush=True)


def pool_requests(np, W, spec):
    """Token ids of the workload's requests: the shared prompt prefix (the
    workload's shared_prefix_tokens) followed by a random tail, each request
    as long as the workload's drawn context length, and longer than the
    prefix."""
    rng = np.random.default_rng(3000 + spec.seed)
    lens = W.draw_lens(spec, np.random.default_rng(spec.seed))
    pre_n = spec.shared_prefix_tokens
    prefix = rng.integers(0, 128000, pre_n, dtype=np.int32)
    reqs = []
    for L in lens:
        tail = rng.integers(0, 128000, max(int(L) - pre_n, 1), dtype=np.int32)
        reqs.append(np.concatenate([prefix, tail])[: max(int(L), pre_n + 1)])
    return reqs


def bench_pool(args, np, pkd, W):
    """Time the host block pool (pa_pool_*) on the workload's requests: one
    episode admits every request (prefix lookup, hashing of every full block,
    block hand-out), then runs --steps decode steps (one appended token per
    request and the batch's block-table export), then frees every request.
    `value` is decode steps per second; admission is reported beside it."""
    import oracle
    spec = W.SPECS[args.workload]
    if not spec.shared_prefix_tokens:      # the long-context workload is the one with a prefix
        spec = W.SPECS[5]
    reqs = pool_requests(np, W, spec)
    B, mbs = len(reqs), spec.max_blocks_per_seq
    need = sum(-(-len(r) // 16) + args.steps // 16 + 2 for r in reqs)
    nb = int(need * 1.2)
    steps = args.steps

    def episode(make, tables):
        p = make()
        t0 = time.perf_counter()
        hits = [p.add_sequence(i, r) for i, r in enumerate(reqs)]
        t1 = time.perf_counter()
        for k in range(steps):
            for i in range(B):
                p.append_token(i, k)
            tables(p)
        t2 = time.perf_counter()
        for i in range(B):
            p.free_sequence(i)
        return t1 - t0, t2 - t1, hits

    nat_tables = lambda p: p.block_table(list(range(B)), mbs, 0)
    for _ in range(max(1, args.warmup // 25)):
        episode(lambda: pkd.BlockPool(nb, 1), nat_tables)
    reps, adm, run = 5, [], []
    for _ in range(reps):
        a, r, hits = episode(lambda: pkd.BlockPool(nb, 1), nat_tables)
        adm.append(a)
        run.append(r)
    prompt_tokens = int(sum(len(r) for r in reqs))
    step_s = min(run) / steps
    rec = {
        "metric": "host block pool decode-step bookkeeping (appends + block-table export)",
        "value": round(1.0 / step_s, 3), "unit": "steps/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int32",
        "data": "synthetic (seeded token ids: shared prompt prefix + random tails)",
        "config": {"workload": spec.name, "op": "block_pool", "requests": B,
                   "prompt_tokens": prompt_tokens, "prefix_tokens_reused": int(sum(hits)),
                   "pool_blocks": nb, "max_blocks_per_seq": mbs,
                   "admit_ms": round(min(adm) * 1e3, 3),
                   "admit_prompt_tokens_per_s": round(prompt_tokens / min(adm), 1)},
        "roofline": None,
        "note": "host code with no GPU kernel: no roofline; best of 5 episodes",
    }
    if not args.no_cpu_baseline:
        ref_steps = max(1, min(steps, 50))
        t0 = time.perf_counter()
        p = oracle.BlockPoolRef(nb, 1)
        for i, r in enumerate(reqs):
            p.add_sequence(i, r.tolist())
        ta = time.perf_counter() - t0
        t1 = time.perf_counter()
        for k in range(ref_steps):
            for i in range(B):
                p.append_token(i, k)
            p.block_table(list(range(B)), mbs, 0)
        tr = time.perf_counter() - t1
        rec["cpu_baseline"] = {"value": round(ref_steps / tr, 3), "unit": "steps/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"one admission ({ta:.1f} s, "
                                         f"{prompt_tokens / ta:.0f} prompt tokens/s) "
                                         f"then {ref_steps} decode steps"}
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the decode path runs whole on one MI355X and "
              "has no multi-GPU mode; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_decode_05_amd as pkd
    from paged_kv_decode_05_amd import workloads as W

    if args.op == "append":
        return bench_append(args, torch, np, pkd, W)
    if args.op == "multi":
        return bench_multi(args, torch, np, pkd, W)
    if args.op == "merge":
        return bench_merge(args, torch, np, pkd, W)
    if args.op == "pool":
        return bench_pool(args, np, pkd, W)

    rec = bench_decode(args, torch, np, pkd, W)
    print(json.dumps(rec), flush=True)


def shape_name(spec):
    """The workload's name without the split it was specified with: the
    split every number was measured with is named beside it."""
    return spec.name.replace("_split512", "")


class DecodeBench:
    """One workload on the GPU: the KV pool rotated over enough copies that the
    Infinity Cache cannot serve repeats, calls marshalled once per split mode,
    HIP events on the launching stream around back-to-back calls."""

    def __init__(self, torch, np, pkd, W, spec):
        self.torch, self.np, self.pkd, self.W = torch, np, pkd, W
        self.spec = spec
        self.wl = W.make_workload(spec)
        self.dev = torch.device("cuda:0")
        t = W.to_device(self.wl, self.dev)
        self.t = t
        pool_bytes = t["k_cache"].numel() * t["k_cache"].element_size() * 2
        self.reps = max(1, math.ceil(3 * MALL_BYTES / pool_bytes))
        self.kcs = [t["k_cache"]] + [t["k_cache"].clone() for _ in range(self.reps - 1)]
        self.vcs = [t["v_cache"]] + [t["v_cache"].clone() for _ in range(self.reps - 1)]
        self.out = torch.empty_like(t["q"])
        self.stream = torch.cuda.current_stream()

    def calls(self, ps):
        pkd, t, torch = self.pkd, self.t, self.torch
        ws = None
        prefix = self.spec.shared_prefix_tokens // 16 if ps == PREFIX else None
        if ps:
            need = (pkd.prefix_workspace_bytes(t["q"], t["k_cache"], t["block_table"]) if prefix is not None
                    else pkd.workspace_bytes(t["q"], t["k_cache"], t["block_table"], ps))
            if need <= 0:
                raise SystemExit(f"no workspace size for mode {mode_name(ps)}")
            ws = torch.empty(need, dtype=torch.uint8, device=self.dev)
            pkd.reset_workspace(ws)
        return [pkd.prepare(t["q"], self.kcs[i], self.vcs[i], t["block_table"], t["context_lens"],
                            float(self.wl.scale), k_scale=t["k_scale"], v_scale=t["v_scale"],
                            partition_size=mode_partition(ps), out=self.out, workspace=ws,
                            stream=self.stream, prefix_blocks=prefix)
                for i in range(self.reps)]

    def time(self, ps, steps, warmup):
        """-> (ms per call, output as float64)"""
        torch = self.torch
        calls = self.calls(ps)
        for i in range(warmup):
            calls[i % self.reps]()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for i in range(steps):
            calls[i % self.reps]()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return (e0.elapsed_time(e1) / steps,
                self.out.float().cpu().numpy().astype(self.np.float64))

    def flush_check(self, ps, n=40):
        """Median time of single calls, each after a 1 GiB write that evicts
        L2 and the Infinity Cache (events around the call only): a
        cross-check of the rotated-pool timing."""
        torch = self.torch
        calls = self.calls(ps)
        scratch = torch.empty(1 << 28, dtype=torch.int32, device=self.dev)
        times = []
        for i in range(n + 3):
            scratch.fill_(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            calls[0]()
            e1.record(self.stream)
            torch.cuda.synchronize()
            if i >= 3:
                times.append(e0.elapsed_time(e1) * 1e3)
        del scratch
        times.sort()
        return times[len(times) // 2]

    def page_read_floor(self):
        """GB/s of a kernel that reads exactly this call's K and V pages (the
        same 16 x head_dim runs, in the same pair-major order, over the same
        rotated pool copies) and does nothing else with them: what the page
        layout and HBM allow for these bytes on this GPU."""
        import ctypes
        np, torch, wl, spec = self.np, self.torch, self.wl, self.spec
        if not os.path.exists(PROBES):
            return None
        lib = ctypes.CDLL(PROBES)
        lib.pa_probe_page_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_void_p]
        page = 16 * spec.head_dim * ELEM.get(spec.kv_dtype, 2)
        if page % 1024:
            return None
        H = spec.num_kv_heads
        cache_bytes = wl.num_blocks * H * page + page          # + the spare block
        offs = []
        for b in range(spec.batch):
            for g in range(H):
                for j in range(-(-int(wl.context_lens[b]) // 16)):
                    blk = int(wl.block_table[b, j])
                    o = (blk * H + g) * page
                    offs.append(o)                  # K page
                    offs.append(cache_bytes + o)    # V page
        offs = np.asarray(offs, dtype=np.uint64)
        per = 2 * cache_bytes
        reps = self.reps
        buf = torch.empty(per * reps, dtype=torch.uint8, device=self.dev)
        assert offs.max() + page <= per
        lists = [torch.from_numpy((offs + r * per).astype(np.int64)).to(self.dev) for r in range(reps)]
        sink = torch.zeros(4, dtype=torch.int32, device=self.dev)
        s = self.stream
        n = len(offs)
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        best = 0.0
        for blocks in (cus, 2 * cus):
            for i in range(10):
                assert lib.pa_probe_page_read(buf.data_ptr(), lists[i % reps].data_ptr(), n,
                                              page // 1024, sink.data_ptr(), blocks,
                                              s.cuda_stream) == 0
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            k = 200
            e0.record(s)
            for i in range(k):
                lib.pa_probe_page_read(buf.data_ptr(), lists[i % reps].data_ptr(), n, page // 1024,
                                       sink.data_ptr(), blocks, s.cuda_stream)
            e1.record(s)
            torch.cuda.synchronize()
            best = max(best, n * page * k / (e0.elapsed_time(e1) / 1e3) / 1e9)
        del buf
        return best


ELEM = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}


def oracle_errors(wl, gpu_out, seqs=None):
    import numpy as np
    import oracle
    s = wl.spec
    ref = oracle.paged_decode_ref(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.context_lens,
                                  wl.scale, s.io_dtype, s.kv_dtype, wl.k_scale, wl.v_scale,
                                  seqs=seqs)
    sel = slice(None) if seqs is None else list(seqs)
    err = np.abs(gpu_out[sel] - ref[sel])
    return float(err.max()), float(err.mean())


# Sequences the per-workload oracle check samples (None: all of them): the
# fp8 B128 and long-context workloads take the oracle seconds per sequence.
ORACLE_SAMPLE = {1: None, 2: None, 3: None, 4: [0, 37, 127], 5: [0, 5]}


def config_record(args, torch, np, pkd, W, k):
    """Every split mode the library offers for workload k, timed; the best
    one's numbers, and its output against the float64 oracle."""
    spec = W.SPECS[k]
    bench = DecodeBench(torch, np, pkd, W, spec)
    modes = [spec.partition_size, pkd.SPLIT_BALANCED] + ([512] if spec.partition_size == 0 else []) \
        + ([PREFIX] if spec.shared_prefix_tokens else [])
    steps = max(50, args.steps // 4)
    timed = {m: bench.time(m, steps, max(10, args.warmup // 2)) for m in modes}
    best = min(timed, key=lambda m: timed[m][0])
    ms, out = timed[best]
    wl = bench.wl
    logical, unique = wl.kv_bytes_logical(), wl.kv_bytes_unique()
    mx, mean = oracle_errors(wl, out, ORACLE_SAMPLE[k])
    floor = None if args.no_stream_ceiling else bench.page_read_floor()
    rec = {
        "workload": shape_name(spec), "spec_partition_size": spec.partition_size,
        "mode": mode_name(best), "us_per_call": round(ms * 1e3, 3),
        "kv_bytes_logical": logical, "kv_bytes_unique": unique,
        "GBps_logical": round(logical / (ms / 1e3) / 1e9, 1),
        "GBps_unique": round(unique / (ms / 1e3) / 1e9, 1),
        "pct_peak_logical": round(100.0 * logical / (ms / 1e3) / 1e9 / PEAK_GBPS, 2),
        "pct_peak_unique": round(100.0 * unique / (ms / 1e3) / 1e9 / PEAK_GBPS, 2),
        "seq_tokens_per_s": round(int(wl.context_lens.astype(np.int64).sum()) / (ms / 1e3), 1),
        "max_abs_vs_oracle": mx, "mean_abs_vs_oracle": mean,
        "oracle_sequences": "all" if ORACLE_SAMPLE[k] is None else ORACLE_SAMPLE[k],
        "modes_us": {mode_name(m): round(v[0] * 1e3, 3) for m, v in timed.items()},
        # a kernel that reads exactly the call's pages (every sequence's, in
        # pair order) and nothing else: logical KV bytes per second
        "page_read_floor_GBps": None if floor is None else round(floor, 1),
        "pct_page_read_floor": None if floor is None else round(100.0 * logical / (ms / 1e3) / 1e9 / floor, 2),
    }
    del bench
    torch.cuda.empty_cache()
    return rec


def bench_decode(args, torch, np, pkd, W):
    spec = W.SPECS[args.workload]
    bench = DecodeBench(torch, np, pkd, W, spec)
    wl = bench.wl

    if args.partition_size is not None:
        modes = [args.partition_size]
    elif args.split == "balanced":
        modes = [pkd.SPLIT_BALANCED, spec.partition_size]
    elif args.split == "prefix":
        if not spec.shared_prefix_tokens:
            raise SystemExit(f"workload {args.workload} has no shared prefix")
        modes = [PREFIX, pkd.SPLIT_BALANCED, spec.partition_size]
    else:
        modes = [spec.partition_size, pkd.SPLIT_BALANCED]
        if spec.partition_size == 0:
            # one pass leaves a long sequence to one workgroup, which streams
            # at a per-CU rate; 512-token partitions are timed beside it
            modes.append(512)
        if spec.shared_prefix_tokens:
            modes.append(PREFIX)
    ps = modes[0]   # --pmc-pass profiles this one

    if args.pmc_pass:
        calls = bench.calls(ps)
        src = torch.ones(1 << 28, dtype=torch.int32, device=bench.dev)      # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        for i in range(20):
            calls[i % bench.reps]()
        torch.cuda.synchronize()
        sys.exit(0)

    timed = {}
    for mode in modes:
        timed[mode] = bench.time(mode, args.steps, args.warmup)
    if args.split == "auto" and args.partition_size is None:
        ps = min(timed, key=lambda m: timed[m][0])
    ms, gpu_out = timed[ps]

    kv_bytes = wl.kv_bytes_logical()
    kv_unique = wl.kv_bytes_unique()
    gbps = kv_bytes / (ms / 1e3) / 1e9
    sum_tokens = int(wl.context_lens.astype(np.int64).sum())
    traffic = traffic_from_profile(spec.name, ps)
    ceiling = None if args.no_stream_ceiling else stream_read_ceiling(torch)
    floor = None if args.no_stream_ceiling else bench.page_read_floor()
    flushed_us = None if args.no_flush_check else bench.flush_check(ps)

    rec = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "f16", "bf16": "bf16"}[spec.io_dtype]
                 + ("" if spec.kv_dtype == spec.io_dtype else "+fp8_e4m3_kv"),
        "data": "synthetic (seeded N(0,1) q/K/V, seeded lengths and block permutation)",
        "config": {
            "workload": shape_name(spec),
            "batch": spec.batch,
            "q_heads": spec.num_q_heads,
            "kv_heads": spec.num_kv_heads,
            "head_dim": spec.head_dim,
            "block_size": 16,
            "context_lens": f"{spec.lens[0]} {list(spec.lens[1:])}",
            "sum_context_tokens": sum_tokens,
            "spec_partition_size": spec.partition_size,
            "split": mode_name(ps),
            "partition_size": mode_partition(ps),
            "prefix_blocks": spec.shared_prefix_tokens // 16 if ps == PREFIX else None,
            "split_choice": ("the faster of the modes timed (listed under modes), all of which "
                             "compute the same result and meet the same parity bar"
                             if args.split == "auto" and args.partition_size is None
                             else "fixed by the command line"),
            "kv_bytes_per_step": kv_bytes,
            "kv_bytes_unique_per_step": kv_unique,
            "pool_copies_rotated": bench.reps,
        },
        "pct_hbm_peak": round(100.0 * gbps / PEAK_GBPS, 2),
        "pct_hbm_peak_unique_bytes": round(100.0 * kv_unique / (ms / 1e3) / 1e9 / PEAK_GBPS, 2),
        "seq_tokens_per_s": round(sum_tokens / (ms / 1e3), 1),
        "seqs_per_s": round(spec.batch / (ms / 1e3), 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbps, 2),
            "peak": PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gbps / PEAK_GBPS, 4),
            "traffic": traffic,
        },
        "stream_read_ceiling_GBps": None if ceiling is None else round(ceiling, 1),
        "pct_stream_ceiling": None if ceiling is None else round(100.0 * gbps / ceiling, 2),
        "page_read_floor_GBps": None if floor is None else round(floor, 1),
        "pct_page_read_floor": None if floor is None else round(100.0 * gbps / floor, 2),
        "flush_check": None if flushed_us is None else {
            "us_median_single_call_after_cache_eviction": round(flushed_us, 2),
            "GBps": round(kv_bytes / (flushed_us / 1e6) / 1e9, 2), "mode": mode_name(ps)},
        "modes": {mode_name(m): {"partition_size": mode_partition(m), "ms_per_step": round(v[0], 6),
                                 "GBps": round(kv_bytes / (v[0] / 1e3) / 1e9, 2),
                                 "max_abs_vs_value_mode": float(np.abs(v[1] - gpu_out).max())}
                  for m, v in timed.items()},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, gpu_out, args.cpu_seconds)
    del bench
    torch.cuda.empty_cache()
    if not args.no_configs:
        rec["configs"] = [config_record(args, torch, np, pkd, W, k) for k in sorted(W.SPECS)]
    return rec


if __name__ == "__main__":
    main()
