"""Compile the HIP sources for gfx950 with hipcc (in-tree shared libraries).

    python -m paged_kv_decode_05_amd.build
"""
import os
import subprocess
import sys

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


def build_one(srcs, dst, verbose=False):
    if isinstance(srcs, str):
        srcs = [srcs]
    tmp = dst + ".tmp"
    cmd = [HIPCC, *COMMON, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {srcs}:\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, dst)
    return dst


def build_all(verbose=False):
    return [build_one(s, d, verbose) for s, d in TARGETS]


if __name__ == "__main__":
    for p in build_all(verbose="-v" in sys.argv):
        print("built", p)
