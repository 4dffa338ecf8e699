"""Randomised parity sweep on an MI355X: seeded configurations drawn over the
whole contract (head_dim 64/128, every io/KV dtype pair, 1-8 KV heads, groups
of 1-16, batches of 1-12, tables of 1-80 blocks, lengths 0, 1, a full table,
a whole number of blocks or anything in between, one to eight new tokens,
one pass, 16- to 512-token partitions - more than 16 of them per sequence
takes the two-level merge - and the balanced split when the rows fit one
tile) against the float64 oracle, output and log-sum-exp. Same bar as the
other parity tests: max-abs 1e-2 / mean-abs 1e-3, fp8 caches 3e-2 / 3e-3;
lse within 5e-3, -inf exactly where the oracle has it."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_05_amd as pkd
from paged_kv_decode_05_amd import workloads as W
from tests.gpu_util import errors, to_device, to_f64
from tests.test_gpu_parity import tol as parity_tol

pytestmark = pytest.mark.gpu

DTYPES = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f16", "fp8_e4m3"),
          ("bf16", "fp8_e4m3")]


def config(seed):
    rng = np.random.default_rng(7000 + seed)
    io, kv = DTYPES[int(rng.integers(len(DTYPES)))]
    D = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.integers(1, 17))
    B = int(rng.integers(1, 13))
    mbs = int(rng.integers(1, 81))
    top = mbs * W.BLOCK_SIZE
    lens = []
    for kind in rng.integers(0, 5, size=B):
        lens.append([0, 1, top, int(rng.integers(1, top + 1)),
                     W.BLOCK_SIZE * int(rng.integers(1, mbs + 1))][int(kind)])
    T = int(rng.choice([1, 1, 1, 2, 3, 5, 8]))
    ps = int(rng.choice([0, 16, 48, 64, 512]))
    if G * T <= 16 and rng.random() < 0.4:
        ps = -1   # balanced split
    needed = sum(-(-L // W.BLOCK_SIZE) for L in lens)
    spec = W.Spec(f"rand{seed}_{io}_{kv}_d{D}_h{G * hkv}kv{hkv}_b{B}_T{T}_ps{ps}", B, G * hkv,
                  hkv, D, io, kv, ("fixed", lens), mbs, ("fixed", int(1.3 * needed) + 2), ps, 0,
                  7000 + seed)
    return spec, T


@pytest.mark.parametrize("seed", range(96))
def test_random_configuration(seed):
    spec, T = config(seed)
    print(f"case {spec.name} lens={spec.lens[1]}", flush=True)
    wl = W.make_workload(spec)
    t = to_device(wl)
    if T == 1:
        qt = t["q"]
        exp, rlse = oracle.paged_decode_ref(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                            wl.context_lens, wl.scale, spec.io_dtype,
                                            spec.kv_dtype, wl.k_scale, wl.v_scale, return_lse=True)
    else:
        q = W.multi_query(wl, T)
        qt = W.storage_tensor(q, spec.io_dtype).cuda()
        exp, rlse = oracle.multi_query_ref(q, wl.k_cache, wl.v_cache, wl.block_table,
                                           wl.context_lens, wl.scale, spec.io_dtype,
                                           spec.kv_dtype, wl.k_scale, wl.v_scale, return_lse=True)
    lse = torch.full(tuple(qt.shape[:-1]), float("nan"), device="cuda")
    out = pkd.decode(qt, t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"],
                     float(wl.scale), k_scale=t["k_scale"], v_scale=t["v_scale"],
                     partition_size=spec.partition_size, lse_out=lse)
    torch.cuda.synchronize()
    got = to_f64(out)
    assert np.isfinite(got).all(), spec.name
    mx, mean = errors(got, exp)
    tol = parity_tol(spec)
    print(f"  max-abs {mx:.3e} mean-abs {mean:.3e}", flush=True)
    assert mx <= tol["max"] and mean <= tol["mean"], (spec.name, mx, mean)
    l = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(l), np.isneginf(rlse)), spec.name
    fin = np.isfinite(rlse)
    assert np.isfinite(l[fin]).all()
    if fin.any():
        assert np.abs(l[fin] - rlse[fin]).max() <= 5e-3, spec.name
