"""pa_lse_merge (decode-context-parallel merge of position shards) against
the oracle on an MI355X, and the single-GPU half of decode context
parallelism end to end: every sequence's positions cut into shards, one
pa_decode per shard with lse_out, merged, compared with the unsharded
oracle decode (bar: max-abs <= 1e-2, mean-abs <= 1e-3; fp8 caches 3e-2)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_05_amd as pkd
from paged_kv_decode_05_amd import workloads as W
from paged_kv_decode_05_amd.workloads import storage_tensor
from tests.gpu_util import to_device, to_f64
from tests.test_gpu_parity import check, ref
from tests.test_oracle_merge_pins import shard_bounds

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("S,D", [(1, 128), (3, 64), (8, 128), (37, 16)])
def test_merge_matches_oracle(dtype, S, D):
    rng = np.random.default_rng(S * 100 + D)
    rows = 301
    o = rng.standard_normal((S, rows, D)).astype(np.float32)
    lse = (rng.standard_normal((S, rows)) * 4).astype(np.float32)
    lse[rng.random((S, rows)) < 0.2] = -np.inf           # empty shards
    lse[:, 7] = -np.inf                                   # a row with no tokens at all
    if S > 1:
        lse[1, 11] = np.nan                               # an out-of-contract shard
    raw = W._to_storage(o, dtype)
    out_t = pkd.lse_merge(storage_tensor(raw, dtype).cuda(), torch.from_numpy(lse).cuda(),
                          lse_out=(lse_t := torch.empty(rows, device="cuda")))
    torch.cuda.synchronize()
    want, wlse = oracle.shard_merge_ref(raw, lse, dtype)
    got = to_f64(out_t)
    glse = lse_t.cpu().double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want)) and np.array_equal(np.isnan(glse), np.isnan(wlse))
    ok = ~np.isnan(want)
    tol = 1e-5 if dtype == "f32" else 1e-2
    err = np.abs(got[ok] - want[ok])
    print(f"  merge {dtype} S{S} D{D}: max-abs {err.max():.2e}", flush=True)
    assert err.max() <= tol * max(1.0, np.abs(want[ok]).max() / 4)
    fin = np.isfinite(wlse)
    assert np.array_equal(np.isneginf(glse), np.isneginf(wlse))
    assert np.abs(glse[fin] - wlse[fin]).max() <= 1e-5 * max(1.0, np.abs(wlse[fin]).max())
    assert np.array_equal(got[7], np.zeros(D))
    if S == 1:
        assert np.array_equal(got[ok], want[ok])           # one shard: the input itself


@pytest.mark.parametrize("k,S", [(1, 2), (3, 4), (4, 3), (5, 8)])
def test_decode_context_parallel_on_one_gpu(k, S):
    spec = W.SPECS[k] if k == 1 else W.small_variant(W.SPECS[k], 5, ("uniform", 40, 3000),
                                                      max_blocks_per_seq=190)
    wl = W.make_workload(spec)
    t = to_device(wl)
    B, Hq, D = wl.q.shape
    outs, lses = [], []
    for s in range(S):
        bt = np.zeros_like(wl.block_table)
        lens = np.zeros(B, dtype=np.int32)
        for b in range(B):
            lo, hi = shard_bounds(int(wl.context_lens[b]), S)[s]
            n = -(-hi // 16) - lo // 16
            bt[b, :n] = wl.block_table[b, lo // 16: lo // 16 + n]
            lens[b] = hi - lo
        lse_s = torch.empty((B, Hq), device="cuda")
        o = pkd.decode(t["q"], t["k_cache"], t["v_cache"], torch.from_numpy(bt).cuda(),
                       torch.from_numpy(lens).cuda(), float(wl.scale), k_scale=t["k_scale"],
                       v_scale=t["v_scale"], partition_size=spec.partition_size, lse_out=lse_s)
        outs.append(o)
        lses.append(lse_s)
    merged = pkd.lse_merge(torch.stack(outs).contiguous(), torch.stack(lses).contiguous())
    torch.cuda.synchronize()
    check(wl, to_f64(merged), ref(wl), label=f"decode-CP w{k} S{S}")
