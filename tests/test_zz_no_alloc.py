"""pa_decode_noalloc (the entry point for callers that cannot allocate)
against pa_decode with a caller's workspace, through the C ABI, on an MI355X.

Both run the same kernels; only where the partial results and counters live
differs (the library's per-GPU scratch with a fixed counter region, or the
caller's workspace), so the outputs must be bit-identical, and both must meet
the oracle bar (max-abs <= 1e-2, mean-abs <= 1e-3 for f16/bf16 caches; fp8
max-abs <= 3e-2). Calls follow each other on the shared scratch: a larger
call, then a smaller one, then the larger again, in every split mode.
"""
import numpy as np
import pytest
import torch

import paged_kv_decode_05_amd as pkd
from paged_kv_decode_05_amd import workloads as W
from tests.gpu_util import to_device, to_f64
from tests.test_gpu_parity import check, ref

pytestmark = pytest.mark.gpu

BAL = pkd.SPLIT_BALANCED


def both(wl, ps):
    t = to_device(wl)
    args = (t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"],
            float(wl.scale))
    kw = dict(k_scale=t["k_scale"], v_scale=t["v_scale"], partition_size=ps)
    B, Hq = wl.q.shape[:2]
    lse_a = torch.full((B, Hq), float("nan"), device="cuda")
    lse_b = torch.full((B, Hq), float("nan"), device="cuda")
    a = pkd.decode_noalloc(*args, lse_out=lse_a, **kw)
    b = pkd.decode(*args, lse_out=lse_b, **kw)
    torch.cuda.synchronize()
    return a, b, lse_a, lse_b


@pytest.mark.parametrize("ps", [512, 64, BAL, 0])
def test_noalloc_equals_decode_on_calls_of_falling_and_rising_size(ps):
    big = W.small_variant(W.SPECS[3], 8, ("uniform", 100, 3000))
    small = W.small_variant(W.SPECS[3], 3, ("uniform", 600, 2000))
    fp8 = W.small_variant(W.SPECS[4], 5, ("uniform", 1, 2500))
    for i, spec in enumerate((big, small, big, fp8, small)):
        print(f"case noalloc ps={ps} call {i}: {spec.name} batch {spec.batch}", flush=True)
        wl = W.make_workload(spec, seed=40 + i)
        a, b, la, lb = both(wl, ps)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (ps, i)
        assert torch.equal(la.view(torch.int32), lb.view(torch.int32)), (ps, i)
        check(wl, to_f64(a), ref(wl), label=f"noalloc ps={ps} call {i}")


def test_noalloc_long_context_two_level_merge_then_smaller_call():
    # 16-token partitions of long sequences: more than 16 partitions per
    # sequence, so the merge-group counters in the fixed counter region are
    # used too (188 partitions in groups of 16: 6.6 MB of partial results);
    # then a small one-level call on the same scratch
    long_ = W.small_variant(W.SPECS[5], 2, ("loguniform", 600, 3000))
    short = W.small_variant(W.SPECS[3], 4, ("uniform", 16, 500))
    for i, (spec, ps) in enumerate(((long_, 16), (short, 512), (long_, 16))):
        print(f"case noalloc two-level call {i}: {spec.name} ps={ps}", flush=True)
        wl = W.make_workload(spec, seed=60 + i)
        a, b, _, _ = both(wl, ps)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), i
        check(wl, to_f64(a), ref(wl), label=f"noalloc two-level call {i}")


def test_noalloc_refuses_a_call_beyond_its_scratch():
    spec = W.small_variant(W.SPECS[3], 2, ("uniform", 100, 200))
    wl = W.make_workload(spec)
    t = to_device(wl)
    # a table of 65536 blocks per sequence at 16-token partitions: 4096
    # partitions x 7 rows x 129 floats per pair, far beyond the scratch
    wide = torch.zeros((2, 65536), dtype=torch.int32, device="cuda")
    with pytest.raises(pkd.PaError) as e:
        pkd.decode_noalloc(t["q"], t["k_cache"], t["v_cache"], wide, t["context_lens"],
                           float(wl.scale), partition_size=16)
    assert e.value.status == 9
