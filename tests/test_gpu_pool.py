"""Block tables from the native block pool, read by the decode kernels on an
MI355X: requests behind shared prompt prefixes share physical blocks (the
pool's prefix reuse), and a few serving steps (pool append, paged KV append,
decode) match the oracle doing the same steps on the same tables. Slots no
sequence owns hold NaN, so a read outside the pool's tables shows."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_05_amd as pkd
from paged_kv_decode_05_amd import workloads as W
from paged_kv_decode_05_amd.workloads import storage_tensor
from tests.gpu_util import to_f64
from tests.test_gpu_append import new_rows
from tests.test_gpu_parity import check, ref

pytestmark = pytest.mark.gpu

MBS = 96


def pool_workload(io, kv, ps, seed):
    """Six requests: four behind one 512-token prompt prefix, two behind its
    first 300 tokens, each with its own tail; caches drawn per physical
    block, NaN wherever no sequence has a token."""
    rng = np.random.default_rng(seed)
    nb, B, Hq, Hkv, D = 400, 6, 8, 2, 128
    pool = pkd.BlockPool(nb, seed)
    prefix = rng.integers(0, 32000, 512).tolist()
    hits = []
    for s in range(B):
        tail = rng.integers(0, 32000, int(rng.integers(1, 700))).tolist()
        hits.append(pool.add_sequence(s, (prefix if s % 3 else prefix[:300]) + tail))
    assert hits == [0, 288, 512, 288, 512, 512]
    table, lens = pool.block_table(list(range(B)), MBS, pad=0)
    spec = W.Spec(f"pool_{io}_{kv}_{ps}", B, Hq, Hkv, D, io, kv, ("fixed", lens.tolist()), MBS,
                  ("fixed", nb), ps, 0, seed)
    x = 16 // oracle.ELEM_BYTES[kv]
    k_cache, k_scale = W._pool_draw(rng, (nb, Hkv, D // x, 16, x), kv)
    v_cache, v_scale = W._pool_draw(rng, (nb, Hkv, D, 16), kv)
    q = W._to_storage(W._normal(rng, (B, Hq, D)), io)
    wl = W.Workload(spec=spec, context_lens=lens, block_table=table, num_blocks=nb,
                    spare_block=0, q=q, k_cache=k_cache, v_cache=v_cache,
                    scale=np.float32(1 / np.sqrt(D)), k_scale=k_scale, v_scale=v_scale)
    poison_unowned(wl, pool)
    return wl, pool


def poison_unowned(wl, pool):
    """NaN in every slot past the owning sequence's length, and in every block
    the pool has not handed out."""
    owned = {}
    for b in range(wl.spec.batch):
        L = int(wl.context_lens[b])
        for j in range(-(-L // 16)):
            blk = int(wl.block_table[b, j])
            owned[blk] = max(owned.get(blk, 0), min(16, L - 16 * j))
    kv = wl.spec.kv_dtype
    for blk in range(wl.num_blocks):
        n = owned.get(blk, 0)
        if n < 16:
            W._nan_fill(wl.k_cache, kv, (blk, slice(None), slice(None), slice(n, None)))
            W._nan_fill(wl.v_cache, kv, (blk, slice(None), slice(None), slice(n, None)))


@pytest.mark.parametrize("io,kv,ps", [("bf16", "bf16", pkd.SPLIT_BALANCED),
                                      ("f16", "fp8_e4m3", 512), ("f16", "f16", 0)])
def test_pool_tables_serving_steps(io, kv, ps):
    wl, pool = pool_workload(io, kv, ps, seed=21)
    print(f"case {wl.spec.name}", flush=True)
    # sequences behind one prefix point at the same physical blocks
    assert (wl.block_table[1, :32] == wl.block_table[2, :32]).all()
    assert (wl.block_table[0, :18] == wl.block_table[3, :18]).all()
    t = W.to_device(wl)
    out = pkd.decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"],
                     float(wl.scale), k_scale=t["k_scale"], v_scale=t["v_scale"],
                     partition_size=ps)
    torch.cuda.synchronize()
    check(wl, to_f64(out), ref(wl), label=f"pool tables {io}/{kv} ps{ps}")

    rng = np.random.default_rng(5)
    B, Hkv = wl.spec.batch, wl.spec.num_kv_heads
    ks = wl.k_scale if kv == "fp8_e4m3" else None
    vs = wl.v_scale if kv == "fp8_e4m3" else None
    for step in range(20):
        for s in range(B):
            pool.append_token(s, int(rng.integers(0, 32000)))
        table, lens = pool.block_table(list(range(B)), MBS, pad=0)
        pos = (lens - 1).astype(np.int32)
        k_new, v_new = new_rows(rng, B, Hkv, wl.spec.head_dim, io)
        bt = torch.from_numpy(table).cuda()
        pkd.kv_append(storage_tensor(k_new, io).cuda(), storage_tensor(v_new, io).cuda(),
                      torch.from_numpy(pos).cuda(), bt, t["k_cache"], t["v_cache"],
                      k_scale=t["k_scale"], v_scale=t["v_scale"])
        wl.k_cache, wl.v_cache = oracle.kv_append_ref(wl.k_cache, wl.v_cache, k_new, v_new,
                                                      table, pos, io, kv, ks, vs)
        wl.block_table, wl.context_lens = table, lens
        if step % 5 == 4:
            out = pkd.decode(t["q"], t["k_cache"], t["v_cache"], bt, torch.from_numpy(lens).cuda(),
                             float(wl.scale), k_scale=t["k_scale"], v_scale=t["v_scale"],
                             partition_size=ps)
            torch.cuda.synchronize()
            check(wl, to_f64(out), ref(wl), label=f"step {step} {io}/{kv} ps{ps}")


@pytest.mark.parametrize("io,kv,ps", [("bf16", "bf16", 512), ("f16", "fp8_e4m3", 0)])
def test_pool_tables_speculative_verify_steps(io, kv, ps):
    """A verify loop on pool-built tables: each step the pool takes four
    drafted tokens per request, pa_kv_append writes their K/V (one call per
    token), and pa_decode_multi attends with the four new tokens causal
    among themselves; the oracle does the same steps."""
    T = 4
    wl, pool = pool_workload(io, kv, ps, seed=33)
    t = W.to_device(wl)
    rng = np.random.default_rng(8)
    B, Hkv = wl.spec.batch, wl.spec.num_kv_heads
    ks = wl.k_scale if kv == "fp8_e4m3" else None
    vs = wl.v_scale if kv == "fp8_e4m3" else None
    print(f"case verify {io}/{kv} ps{ps}", flush=True)
    for step in range(3):
        for i in range(T):
            for s in range(B):
                pool.append_token(s, int(rng.integers(0, 32000)))
            table, lens = pool.block_table(list(range(B)), MBS, pad=0)
            pos = (lens - 1).astype(np.int32)
            k_new, v_new = new_rows(rng, B, Hkv, wl.spec.head_dim, io)
            bt = torch.from_numpy(table).cuda()
            pkd.kv_append(storage_tensor(k_new, io).cuda(), storage_tensor(v_new, io).cuda(),
                          torch.from_numpy(pos).cuda(), bt, t["k_cache"], t["v_cache"],
                          k_scale=t["k_scale"], v_scale=t["v_scale"])
            wl.k_cache, wl.v_cache = oracle.kv_append_ref(wl.k_cache, wl.v_cache, k_new, v_new,
                                                          table, pos, io, kv, ks, vs)
        wl.block_table, wl.context_lens = table, lens
        q = W.multi_query(wl, T, seed=100 + step)
        out = pkd.decode(storage_tensor(q, io).cuda(), t["k_cache"], t["v_cache"], bt,
                         torch.from_numpy(lens).cuda(), float(wl.scale), k_scale=t["k_scale"],
                         v_scale=t["v_scale"], partition_size=ps)
        torch.cuda.synchronize()
        exp = oracle.multi_query_ref(q, wl.k_cache, wl.v_cache, table, lens, wl.scale, io, kv,
                                     ks, vs)
        check(wl, to_f64(out), exp, label=f"verify step {step} {io}/{kv} ps{ps}")


def _rows(wl, rows):
    """The workload restricted to some of its sequences (same caches)."""
    import dataclasses
    rows = list(rows)
    spec = dataclasses.replace(wl.spec, batch=len(rows),
                               lens=("fixed", [int(wl.context_lens[r]) for r in rows]))
    return dataclasses.replace(wl, spec=spec, context_lens=wl.context_lens[rows].copy(),
                               block_table=wl.block_table[rows].copy(), q=wl.q[rows].copy())


@pytest.mark.parametrize("io,kv", [("bf16", "bf16"), ("f16", "fp8_e4m3")])
def test_shared_prefix_decode_with_the_pools_prefix(io, kv):
    # the pool reports the blocks a set of its sequences shares; declared to
    # the shared-prefix decode, they are read once for the whole batch
    wl, pool = pool_workload(io, kv, pkd.SPLIT_BALANCED, 41)
    for rows in (range(6), (1, 2, 4, 5)):
        sub = _rows(wl, rows)
        P = pool.shared_prefix(list(rows))
        assert P >= (32 if len(sub.context_lens) == 4 else 18)
        print(f"case pool shared prefix {io}/{kv} rows {list(rows)} P={P}", flush=True)
        t = W.to_device(sub)
        out = pkd.decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"],
                         float(sub.scale), k_scale=t["k_scale"], v_scale=t["v_scale"],
                         partition_size=pkd.SPLIT_BALANCED, prefix_blocks=P)
        torch.cuda.synchronize()
        check(sub, to_f64(out), ref(sub), label=f"pool prefix {list(rows)}")
    pool.close()
