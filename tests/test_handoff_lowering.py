"""The split-K hand-off between workgroups (partials stored, a counter bumped,
the last piece merging) uses no fences: partials are written and read with
SC1 buffer accesses, the same instruction the compiler emits for relaxed
agent-scope atomic stores and loads; every wave waits for its stores
(s_waitcnt vmcnt(0)) before the workgroup's counter increment. This test
compiles the product's helpers (csrc/pa_tiles.h) and the compiler's own
release/acquire increments for gfx950 and checks the claim the design rests
on: the release/acquire pair is exactly the product's sequence plus an L2
writeback (buffer_wbl2) before the increment and an L2 invalidate
(buffer_inv) after it, which act only on data moved by ordinary accesses.
CPU only: hipcc cross-compiles; nothing is launched."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "probes", "handoff_lowering.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not installed")
    out = str(tmp_path_factory.mktemp("handoff") / "handoff.s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "paged_kv_decode_05_amd", "csrc"), SRC, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    text = open(out).read()
    bodies = {}
    for name in ("handoff_product", "handoff_release", "handoff_acquire"):
        m = re.search(r"^(_Z\d+" + name + r"\w*):.*?\n(.*?)s_endpgm", text, re.S | re.M)
        assert m, name
        bodies[name] = [l.strip() for l in m.group(2).splitlines()
                        if l.strip() and not l.strip().startswith((";", "."))]
    return bodies


def first(lines, pattern, start=0):
    for i in range(start, len(lines)):
        if re.search(pattern, lines[i]):
            return i
    return -1


def test_release_and_acquire_add_only_l2_writeback_and_invalidate(asm):
    rel, acq = asm["handoff_release"], asm["handoff_acquire"]
    a = first(rel, r"global_atomic_add")
    w = first(rel, r"^buffer_wbl2 sc1")
    assert 0 <= w < first(rel, r"s_waitcnt vmcnt\(0\)", w) < a
    a = first(acq, r"global_atomic_add")
    i = first(acq, r"^buffer_inv sc1", a)
    assert a < first(acq, r"s_waitcnt vmcnt\(0\)", a) < i < first(acq, r"global_load_dword", i)


def test_product_handoff_is_that_sequence_without_the_cache_maintenance(asm):
    p = asm["handoff_product"]
    st = first(p, r"buffer_store_dwordx4 .* sc1")
    wait = first(p, r"s_waitcnt vmcnt\(0\)", st)
    bar = first(p, r"s_barrier", wait)
    add = first(p, r"global_atomic_add", bar)
    ld = first(p, r"buffer_load_dwordx4 .* sc1", add)
    assert 0 <= st < wait < bar < add < ld, p
    # the returned count is waited for before the loads are issued
    assert first(p, r"s_waitcnt vmcnt\(0\)", add) < ld
    assert not any(re.search(r"buffer_wbl2|buffer_inv|buffer_wbinvl1", l) for l in p), p
