"""Compile the HIP sources for gfx950 with hipcc (in-tree shared libraries).

    python -m paged_kv_decode_05_amd.build
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
    # keep hipcc from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: the online-softmax rescale
    # multiplies them in place instead of copying through AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
    "-I", os.path.join(HERE, "csrc"),
]

TARGETS = [
    ([os.path.join(HERE, "csrc", n) for n in ("pa_decode.hip", "pa_multi.hip", "pa_append.hip", "pa_merge.hip",
                                                     "block_pool.cpp")],
     os.path.join(HERE, "libpadecode.so")),
    ([os.path.join(ROOT, "tests", "probes", "probes.hip")],
     os.path.join(ROOT, "tests", "probes", "libpaprobes.so")),
]


OBJDIR = os.path.join(ROOT, "_build")


def _run(cmd, what, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {what}:\n{out}")
    if verbose and out.strip():
        print(out)


def _jobs():
    try:
        n = int(os.environ.get("MAX_JOBS", "0"))
    except ValueError:
        n = 0
    return max(1, min(n or (os.cpu_count() or 1), 16))


def build_one(srcs, dst, verbose=False):
    """Compile every source to an object in parallel, then link dst."""
    if isinstance(srcs, str):
        srcs = [srcs]
    os.makedirs(OBJDIR, exist_ok=True)
    stem = os.path.splitext(os.path.basename(dst))[0]
    objs = [os.path.join(OBJDIR, f"{stem}.{os.path.basename(s)}.o") for s in srcs]
    compile_flags = [f for f in COMMON if f != "-shared"]
    with ThreadPoolExecutor(max_workers=_jobs()) as pool:
        futures = [pool.submit(_run, [HIPCC, *compile_flags, "-c", s, "-o", o], s, verbose)
                   for s, o in zip(srcs, objs)]
        for f in futures:
            f.result()
    tmp = dst + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], dst, verbose)
    os.replace(tmp, dst)
    return dst


def build_all(verbose=False):
    return [build_one(s, d, verbose) for s, d in TARGETS]


if __name__ == "__main__":
    for p in build_all(verbose="-v" in sys.argv):
        print("built", p)
