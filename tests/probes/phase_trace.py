"""Per-workgroup phase times of the balanced-split decode kernel, measured on
a traced copy of paged_kv_decode_05_amd/csrc/pa_decode.hip.

    python tests/probes/phase_trace.py build                  # on the CPU
    python tests/probes/phase_trace.py run --workload 3       # on an MI355X

`build` writes the copy to _build/phase_trace/ and compiles it, with the
other sources of the library, into tests/probes/libpatrace.so (the same
flags as paged_kv_decode_05_amd/build.py). The copy adds one kernel argument
(a device array, null unless the host hands one in with
pa_debug_set_trace) and at each phase boundary of the balanced kernel's
single-token path thread 0 of the workgroup stores s_memrealtime (a
constant 100 MHz clock) to trace[8 * workgroup + i]:

    0 entry            1 length scan done      2 streaming done (all waves)
    3 LDS combine done 4 partial stores complete
    5 pieces counted   6 end                   7 pairs merged (a count)

A workgroup that leads no piece stamps 0-2 and 6; one whose pieces are all
whole pairs stamps 0-3 and 6. `run` times the traced library without a trace
(the stamps' own cost), then traces single calls on rotated copies of the
cache (so no call finds the previous one's pages in cache) and prints a
markdown summary: each boundary's median and last time over the workgroups,
the phases of the workgroups that end last, and each XCD's streaming
duration (differences of one workgroup's own stamps).

Not part of the product: nothing in the library, the tests or bench.py loads
libpatrace.so.
"""
import argparse
import math
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

CSRC = os.path.join(ROOT, "paged_kv_decode_05_amd", "csrc")
GEN_DIR = os.path.join(ROOT, "_build", "phase_trace")
LIB = os.path.join(ROOT, "tests", "probes", "libpatrace.so")
SLOTS = 8


def _stamp(i):
    return (f"if (a.trace && threadIdx.x == 0) a.trace[(size_t)blockIdx.x * {SLOTS} + {i}] = "
            "__builtin_amdgcn_s_memrealtime();")


def _patches():
    """(anchor, replacement) pairs; every anchor must occur exactly once."""
    return [
        ("  int32_t prefix_pages; // shared prefix: block-table entries every row shares (0: none)\n",
         "  int32_t prefix_pages; // shared prefix: block-table entries every row shares (0: none)\n"
         "  unsigned long long* trace;\n"),
        ("pa_decode_balanced_kernel(const Params a) {\n",
         "pa_decode_balanced_kernel(const Params a) {\n  " + _stamp(0) + "\n"),
        ("  if (tid == kThreads - 1) sm.pre[B] = before + incl;\n  __syncthreads();\n",
         "  if (tid == kThreads - 1) sm.pre[B] = before + incl;\n  __syncthreads();\n  " + _stamp(1) + "\n"),
        ("  decode_quarter<IO, KV, D, MQ, PFX>(a, sm, ShareOf{wg, N, S}, yq(wu), yq(wu + 1), pg.P);\n"
         "  __syncthreads();\n",
         "  decode_quarter<IO, KV, D, MQ, PFX>(a, sm, ShareOf{wg, N, S}, yq(wu), yq(wu + 1), pg.P);\n"
         "  __syncthreads();\n  " + _stamp(2) + "\n"),
        ("  if (!PFX && lead == 0) return;   // uniform\n",
         "  if (!PFX && lead == 0) {\n    " + _stamp(6) + "\n    return;\n  }\n"),
        ("    lds_barrier();\n    const uint32_t stale = (uint32_t)__builtin_amdgcn_readfirstlane(sm.split[1]);\n",
         "    lds_barrier();\n    " + _stamp(5) +
         "\n    const uint32_t stale = (uint32_t)__builtin_amdgcn_readfirstlane(sm.split[1]);\n"),
        ("    const int m = __builtin_popcount(done);\n    merge_jobs<IO, D, merge_batch<KV>()>(a, sm.red, m, npm,",
         "    const int m = __builtin_popcount(done);\n"
         f"    if (a.trace && threadIdx.x == 0) a.trace[(size_t)blockIdx.x * {SLOTS} + 7] = m;\n"
         "    merge_jobs<IO, D, merge_batch<KV>()>(a, sm.red, m, npm,"),
        ("    combine_pieces<IO, KV, D, MQ, PFX>(a, sm, lead, facts);\n"
         "    if (split == 0) return;   // uniform\n"
         "    __builtin_amdgcn_s_waitcnt(0);   // this wave's partial stores are complete\n"
         "    __syncthreads();\n"
         "    settle_split();\n",
         "    combine_pieces<IO, KV, D, MQ, PFX>(a, sm, lead, facts);\n    " + _stamp(3) + "\n"
         "    if (split == 0) {\n      " + _stamp(6) + "\n      return;\n    }\n"
         "    __builtin_amdgcn_s_waitcnt(0);   // this wave's partial stores are complete\n"
         "    __syncthreads();\n    " + _stamp(4) + "\n"
         "    settle_split();\n    " + _stamp(6) + "\n"),
        ("// prefix_blocks >= 0: the shared-prefix call (balanced split only).\n",
         "unsigned long long* g_trace = nullptr;\n"
         "// prefix_blocks >= 0: the shared-prefix call (balanced split only).\n"),
        ("  prm.prefix_pages = prefix ? prefix_blocks : 0;\n",
         "  prm.prefix_pages = prefix ? prefix_blocks : 0;\n  prm.trace = g_trace;\n"),
    ]


def patched_source():
    """The traced copy of pa_decode.hip (raises if an anchor has moved)."""
    src = open(os.path.join(CSRC, "pa_decode.hip")).read()
    for old, new in _patches():
        n = src.count(old)
        if n != 1:
            raise RuntimeError(f"anchor found {n} times: {old[:70]!r}")
        src = src.replace(old, new)
    i = src.rindex('extern "C" {')
    return (src[:i] + 'extern "C" void pa_debug_set_trace(void* p) { pa::g_trace = (unsigned long long*)p; }\n'
            + src[i:])


def build(verbose=False):
    from paged_kv_decode_05_amd import build as B
    os.makedirs(GEN_DIR, exist_ok=True)
    gen = os.path.join(GEN_DIR, "pa_decode.hip")
    with open(gen, "w") as f:
        f.write(patched_source())
    others = [os.path.join(CSRC, n) for n in ("pa_multi.hip", "pa_append.hip", "pa_merge.hip", "block_pool.cpp")]
    return B.build_one([gen, *others], LIB, verbose)


def run(workload, calls):
    import ctypes
    import numpy as np
    import torch
    import paged_kv_decode_05_amd as pkd
    from paged_kv_decode_05_amd import _lib
    from paged_kv_decode_05_amd import workloads as W

    if not os.path.exists(LIB):
        raise SystemExit(f"{LIB} is not built: python tests/probes/phase_trace.py build")
    lib = _lib.load_library(LIB)
    lib.pa_debug_set_trace.argtypes = [ctypes.c_void_p]
    lib.pa_debug_set_trace.restype = None
    _lib._lib = lib   # the binding's calls below go to the traced library

    spec = W.SPECS[workload]
    wl = W.make_workload(spec)
    t = W.to_device(wl)
    pool = t["k_cache"].numel() * t["k_cache"].element_size() * 2
    reps = max(1, math.ceil(3 * (256 << 20) / pool))
    kcs = [t["k_cache"]] + [t["k_cache"].clone() for _ in range(reps - 1)]
    vcs = [t["v_cache"]] + [t["v_cache"].clone() for _ in range(reps - 1)]
    out = torch.empty_like(t["q"])
    ws = torch.zeros(pkd.workspace_bytes(t["q"], t["k_cache"], t["block_table"], pkd.SPLIT_BALANCED),
                     dtype=torch.uint8, device="cuda")
    fns = [pkd.prepare(t["q"], kcs[i], vcs[i], t["block_table"], t["context_lens"], float(wl.scale),
                       k_scale=t["k_scale"], v_scale=t["v_scale"], partition_size=pkd.SPLIT_BALANCED, out=out,
                       workspace=ws) for i in range(reps)]
    for i in range(30):
        fns[i % reps]()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 300
    e0.record()
    for i in range(n):
        fns[i % reps]()
    e1.record()
    torch.cuda.synchronize()
    us_call = e0.elapsed_time(e1) / n * 1e3

    grid = 4096
    tr = torch.zeros(grid * SLOTS, dtype=torch.int64, device="cuda")
    runs = []
    for c in range(calls):
        tr.zero_()
        torch.cuda.synchronize()
        lib.pa_debug_set_trace(tr.data_ptr())
        fns[(c + 1) % reps]()
        torch.cuda.synchronize()
        lib.pa_debug_set_trace(None)
        a = tr.view(grid, SLOTS).cpu().numpy().astype(np.int64)
        live = np.nonzero(a[:, 0] > 0)[0]
        runs.append((live, a[live]))   # block ids, their stamps
    to_us = lambda x, t0: (x - t0) / 100.0

    print(f"# Balanced-split phases: {spec.name}\n")
    print("Made from the repository root with `python tests/probes/phase_trace.py build` (CPU), then "
          f"`python tests/probes/phase_trace.py run --workload {workload} --calls {calls}` on one MI355X. "
          "Times in us from the first workgroup's entry stamp (s_memrealtime, 10 ns steps).\n")
    print(f"Traced library without a trace: {us_call:.2f} us per call (event loop of {n} calls, "
          f"{reps} cache copies rotated). {len(runs[0][0])} workgroups; {calls} traced calls.\n")
    names = ["entry", "scan done", "streamed", "combined", "stores complete", "counted", "end"]
    print("| boundary | median us (mean over calls) | last us (mean over calls) | workgroups stamping |")
    print("|---|---|---|---|")
    for i, nm in enumerate(names):
        med, last, cnt = [], [], 0
        for _, a in runs:
            t0 = a[:, 0].min()
            v = a[:, i]
            v = v[v > 0]
            if len(v):
                med.append(np.median(to_us(v, t0)))
                last.append(to_us(v, t0).max())
                cnt = len(v)
        if med:
            print(f"| {i} {nm} | {np.mean(med):.2f} | {np.mean(last):.2f} | {cnt} |")
    a = runs[0][1]
    t0 = a[:, 0].min()
    print("\nWorkgroups that end last (first traced call), phase durations in us:\n")
    print("| end | scan | streaming | combine | stores | count | merge | pairs merged |")
    print("|---|---|---|---|---|---|---|---|")

    def ph(r, hi, lo):
        return f"{(r[hi] - r[lo]) / 100.0:.2f}" if r[hi] > 0 and r[lo] > 0 else "-"
    for r in a[np.argsort(-a[:, 6])[:8]]:
        print(f"| {to_us(r[6], t0):.2f} | {ph(r, 1, 0)} | {ph(r, 2, 1)} | {ph(r, 3, 2)} | {ph(r, 4, 3)} | "
              f"{ph(r, 5, 4)} | {ph(r, 6, 5)} | {r[7]} |")
    print("\nStreaming duration (stamp 2 - stamp 1 of each workgroup) by XCD "
          "(workgroup b runs on XCD b mod 8), over all traced calls:\n")
    print("| XCD | mean us | max us |")
    print("|---|---|---|")
    dur = {x: [] for x in range(8)}
    for blocks, a in runs:
        for b, r in zip(blocks, a):
            if r[2] > 0 and r[1] > 0:
                dur[int(b) % 8].append((r[2] - r[1]) / 100.0)
    for x in range(8):
        if dur[x]:
            print(f"| {x} | {np.mean(dur[x]):.2f} | {np.max(dur[x]):.2f} |")


if __name__ == "__main__":
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("step", choices=["build", "run"])
    ap.add_argument("--workload", type=int, default=3, choices=[2, 3, 4])
    ap.add_argument("--calls", type=int, default=8)
    ap.add_argument("-v", action="store_true")
    args = ap.parse_args()
    if args.step == "build":
        print("built", build(args.v))
    else:
        run(args.workload, args.calls)
